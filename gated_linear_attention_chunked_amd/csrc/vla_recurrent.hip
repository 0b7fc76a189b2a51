// vla_recurrent.hip -- token-by-token VLA scan on gfx950.
//
// The rules ("Technical summary: Variational Linear Attention (VLA)",
// sections 2.2-2.3): the inverse penalty A = M^{-1} is kept by a rank-1
// Sherman-Morrison downdate per token (O(d^2)), the gating vector is the unit
// vector along A khat, and the state writes its prediction residual along that
// gate; keys and queries pass through ELU+1 and unit normalisation.
//
// Schedule.  One workgroup per (b, h) chain (NW waves).  A and S live in
// registers: TPR lanes per row, each lane RPT rows x CPT columns (rows
// rg + NRG*r, columns lane + TPR*m).  Per token, using the algebra
//   z = A p,  den = 1 + p.z,  A' khat = A khat - z (z.khat)/den,
//   y = S qhat + (v - S khat)(alphahat . qhat),
// one pass over A and S gives A p, A khat, S khat, S qhat together; two
// row-sums (p.z with z.khat, then |A' khat|^2 with (A' khat).qhat) and one
// exchange of z and alphahat through LDS finish the token.  Feature maps and
// norms of a whole tile of keys and queries are computed up front with wave
// reductions.
//
// Ratio read (RATIO): section 2.3 reads the output as a ratio of
// recurrences, as in standard linear attention, where the denominator
// accumulates like the numerator over a value of 1.  The denominator here is
// a d-vector n that follows the write rule with the value 1,
//   n <- n + (1 - n.khat) alphahat,   y = (S qhat) / (n.qhat),
// and by the same algebra as y, n'.qhat = n.qhat + (1 - n.khat)(alphahat.qhat).
// Every row group keeps its own copy of n (the columns of its lanes), so
// n.khat and n.qhat are lane-group sums like the rows of S khat and S qhat.
#include "device_common.h"
#include "lam_internal.h"

namespace lam {
namespace {

constexpr int TT = 16;

template <int D>
struct VlaShape {
    static constexpr int NW = D <= 32 ? 1 : (D <= 64 ? 2 : 4);
    static constexpr int NT = 64 * NW;
    static constexpr int TPR = D >= 96 ? 16 : 8;
    static constexpr int NRG = NT / TPR;
    static constexpr int RPT = D / NRG;
    static constexpr int CPT = D / TPR;
    static_assert(RPT * NRG == D && CPT * TPR == D, "shape");
};

__device__ __forceinline__ float elu_plus_one(float x) { return x > 0.f ? x + 1.f : expf(x); }

template <typename IO, int D, bool RATIO>
__global__ __launch_bounds__(VlaShape<D>::NT) void vla_recurrent_kernel(VlaArgs a) {
    using Sh = VlaShape<D>;
    constexpr int NW = Sh::NW, NT = Sh::NT, TPR = Sh::TPR, NRG = Sh::NRG, RPT = Sh::RPT,
                  CPT = Sh::CPT;
    const int T = static_cast<int>(a.T), H = static_cast<int>(a.H);
    const int b = blockIdx.x / H, h = blockIdx.x % H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = tid % TPR, rg = tid / TPR;

    __shared__ float sk[TT][D], sq[TT][D], sp[TT][D], sv[TT][D];
    __shared__ float sy[TT][D];
    __shared__ float sz[D], sa[D];
    __shared__ float red1[NW][2], red2[NW][2];

    float A[RPT][CPT], S[RPT][CPT];
    const int64_t sb = (static_cast<int64_t>(b) * H + h) * D * D;
#pragma unroll
    for (int r = 0; r < RPT; ++r)
#pragma unroll
        for (int m = 0; m < CPT; ++m) {
            const int i = rg + NRG * r, j = lr + TPR * m;
            A[r][m] = a.A_in ? a.A_in[sb + i * D + j] : (i == j ? 1.f : 0.f);
            S[r][m] = a.S_in ? a.S_in[sb + i * D + j] : 0.f;
        }
    const int64_t nb = (static_cast<int64_t>(b) * H + h) * D;
    float nrow[CPT];
#pragma unroll
    for (int m = 0; m < CPT; ++m) nrow[m] = (RATIO && a.n_in) ? a.n_in[nb + lr + TPR * m] : 0.f;

    constexpr int SLOTS = (TT * D + NT - 1) / NT;
    float rq[SLOTS], rk[SLOTS], rp[SLOTS], rv[SLOTS];
    auto fetch = [&](int t0) {
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int e = tid + s * NT;
            const int t = e / D, j = e % D, tt = t0 + t;
            const bool ok = e < TT * D && tt < T;
            const int64_t gi = ((static_cast<int64_t>(b) * T + tt) * H + h) * D + j;
            rq[s] = ok ? IO::ld(a.q, gi) : 0.f;
            rk[s] = ok ? IO::ld(a.k, gi) : 0.f;
            rp[s] = ok ? IO::ld(a.p, gi) : 0.f;
            rv[s] = ok ? IO::ld(a.v, gi) : 0.f;
        }
    };

    if (T > 0) fetch(0);
    for (int t0 = 0; t0 < T; t0 += TT) {
        __syncthreads();
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int e = tid + s * NT;
            if (e < TT * D) {
                const int t = e / D, j = e % D;
                sq[t][j] = rq[s];
                sk[t][j] = rk[s];
                sp[t][j] = rp[s];
                sv[t][j] = rv[s];
            }
        }
        __syncthreads();
        if (t0 + TT < T) fetch(t0 + TT);
        const int nt = min(TT, T - t0);

        // feature maps: one wave per token, lanes over channels
        for (int t = wave; t < nt; t += NW) {
            float fk[(D + 63) / 64], fq[(D + 63) / 64];
            float ssk = 0.f, ssq = 0.f;
#pragma unroll
            for (int u = 0; u < (D + 63) / 64; ++u) {
                const int j = lane + 64 * u;
                fk[u] = j < D ? elu_plus_one(sk[t][j]) : 0.f;
                fq[u] = j < D ? elu_plus_one(sq[t][j]) : 0.f;
                ssk = fmaf(fk[u], fk[u], ssk);
                ssq = fmaf(fq[u], fq[u], ssq);
            }
            ssk = group_sum<64>(ssk);
            ssq = group_sum<64>(ssq);
            const float ik = 1.f / sqrtf(ssk), iq = 1.f / sqrtf(ssq);
#pragma unroll
            for (int u = 0; u < (D + 63) / 64; ++u) {
                const int j = lane + 64 * u;
                if (j < D) {
                    sk[t][j] = fk[u] * ik;
                    sq[t][j] = fq[u] * iq;
                }
            }
        }
        __syncthreads();

        for (int t = 0; t < nt; ++t) {
            float zp[RPT], wk[RPT], skr[RPT], sqr[RPT];
            float nk = 0.f, nq = 0.f;  // n.khat, n.qhat (ratio read)
#pragma unroll
            for (int r = 0; r < RPT; ++r) zp[r] = wk[r] = skr[r] = sqr[r] = 0.f;
#pragma unroll
            for (int m = 0; m < CPT; ++m) {
                const int j = lr + TPR * m;
                const float pj = sp[t][j], kj = sk[t][j], qj = sq[t][j];
#pragma unroll
                for (int r = 0; r < RPT; ++r) {
                    zp[r] = fmaf(A[r][m], pj, zp[r]);
                    wk[r] = fmaf(A[r][m], kj, wk[r]);
                    skr[r] = fmaf(S[r][m], kj, skr[r]);
                    sqr[r] = fmaf(S[r][m], qj, sqr[r]);
                }
                if constexpr (RATIO) {
                    nk = fmaf(nrow[m], kj, nk);
                    nq = fmaf(nrow[m], qj, nq);
                }
            }
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                zp[r] = group_sum<TPR>(zp[r]);
                wk[r] = group_sum<TPR>(wk[r]);
                skr[r] = group_sum<TPR>(skr[r]);
                sqr[r] = group_sum<TPR>(sqr[r]);
            }
            if constexpr (RATIO) {
                nk = group_sum<TPR>(nk);
                nq = group_sum<TPR>(nq);
            }
            // row sums p.z and khat.z (one lane per row contributes)
            float pz = 0.f, kz = 0.f;
            if (lr == 0) {
#pragma unroll
                for (int r = 0; r < RPT; ++r) {
                    const int i = rg + NRG * r;
                    pz = fmaf(sp[t][i], zp[r], pz);
                    kz = fmaf(sk[t][i], zp[r], kz);
                }
            }
            pz = group_sum<64>(pz);
            kz = group_sum<64>(kz);
            if constexpr (NW > 1) {
                if (lane == 0) {
                    red1[wave][0] = pz;
                    red1[wave][1] = kz;
                }
                __syncthreads();
                pz = kz = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    pz += red1[w][0];
                    kz += red1[w][1];
                }
            }
            const float den = 1.f + pz;
            const float c = kz / den;
            float av[RPT];
            float aa = 0.f, aq = 0.f;
#pragma unroll
            for (int r = 0; r < RPT; ++r) av[r] = fmaf(-zp[r], c, wk[r]);
            if (lr == 0) {
#pragma unroll
                for (int r = 0; r < RPT; ++r) {
                    const int i = rg + NRG * r;
                    aa = fmaf(av[r], av[r], aa);
                    aq = fmaf(av[r], sq[t][i], aq);
                    sz[i] = zp[r];
                }
            }
            aa = group_sum<64>(aa);
            aq = group_sum<64>(aq);
            if constexpr (NW > 1) {
                if (lane == 0) {
                    red2[wave][0] = aa;
                    red2[wave][1] = aq;
                }
            }
            __syncthreads();
            if constexpr (NW > 1) {
                aa = aq = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    aa += red2[w][0];
                    aq += red2[w][1];
                }
            }
            const float inv = 1.f / sqrtf(aa);
            const float ahq = aq * inv;
            const float rn = 1.f - nk;                                // the denominator's residual
            const float ry = RATIO ? 1.f / fmaf(rn, ahq, nq) : 1.f;  // 1 / (n'.qhat)
            float rr[RPT];
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const int i = rg + NRG * r;
                rr[r] = sv[t][i] - skr[r];
                if (lr == 0) {
                    sy[t][i] = RATIO ? fmaf(rr[r], ahq, sqr[r]) * ry : fmaf(rr[r], ahq, sqr[r]);
                    sa[i] = av[r] * inv;
                }
            }
            // A -= z z^T / den uses z from LDS (written before the last barrier)
            float zr[RPT];
#pragma unroll
            for (int r = 0; r < RPT; ++r) zr[r] = zp[r] / den;
#pragma unroll
            for (int m = 0; m < CPT; ++m) {
                const float zj = sz[lr + TPR * m];
#pragma unroll
                for (int r = 0; r < RPT; ++r) A[r][m] = fmaf(-zr[r], zj, A[r][m]);
            }
            __syncthreads();  // alphahat visible
#pragma unroll
            for (int m = 0; m < CPT; ++m) {
                const float aj = sa[lr + TPR * m];
#pragma unroll
                for (int r = 0; r < RPT; ++r) S[r][m] = fmaf(rr[r], aj, S[r][m]);
                if constexpr (RATIO) nrow[m] = fmaf(rn, aj, nrow[m]);
            }
            __syncthreads();  // sz / sa / red slots free for the next token
        }
        __syncthreads();
        for (int e = tid; e < nt * D; e += NT) {
            const int t = e / D, j = e % D;
            const int64_t gi = ((static_cast<int64_t>(b) * T + t0 + t) * H + h) * D + j;
            IO::st(a.out, gi, sy[t][j]);
        }
    }

#pragma unroll
    for (int r = 0; r < RPT; ++r)
#pragma unroll
        for (int m = 0; m < CPT; ++m) {
            const int i = rg + NRG * r, j = lr + TPR * m;
            if (a.A_out) a.A_out[sb + i * D + j] = A[r][m];
            if (a.S_out) a.S_out[sb + i * D + j] = S[r][m];
        }
    if constexpr (RATIO) __syncthreads();  // every row group has read n_in (n_out may be the same buffer)
    if (RATIO && a.n_out && rg == 0) {
#pragma unroll
        for (int m = 0; m < CPT; ++m) a.n_out[nb + lr + TPR * m] = nrow[m];
    }
}

template <typename IO, int D>
hipError_t launch_d(const VlaArgs &a, hipStream_t stream) {
    const unsigned blocks = static_cast<unsigned>(a.B * a.H);
    if (a.ratio)
        vla_recurrent_kernel<IO, D, true><<<dim3(blocks), dim3(VlaShape<D>::NT), 0, stream>>>(a);
    else
        vla_recurrent_kernel<IO, D, false><<<dim3(blocks), dim3(VlaShape<D>::NT), 0, stream>>>(a);
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

hipError_t launch_vla_recurrent(const VlaArgs &a, hipStream_t stream) {
    return a.dtype == kBF16 ? launch_io<IoBF16>(a, stream) : launch_io<IoF32>(a, stream);
}

}  // namespace lam
