// delta_backward.hip -- backward pass of the delta-rule scan (all four
// variants) on gfx950: the gradients of sum <dout, out> + <dstate_out,
// state_out> with respect to q, k, v, the gates, beta and the initial state.
//
// The forward rule ("Mechanisms, trade-offs and cross-layer routing of
// linear-attention architectures", "Technical details"), per token, with read
// key kk (k, or b * k for Gated DeltaNet-2), target z (v, or w * v) and
// W~ the decayed memory (alpha W, W diag(alpha), or W):
//   r = z - W~ kk;  W_t = W~ + beta r k^T;  y_t = W_t q.
// Its adjoint, with G the adjoint of W_t (dstate_out before the last token),
// for t = T-1 .. 0:
//   G += dout_t q^T;  dq_t = W_t^T dout_t;  g = G k;
//   dbeta_t = r . g;  dz = beta g  (dv = dz, or w * dz and dw = v * dz);
//   dk_t = beta G^T r - beta W~^T g  (Gated DeltaNet-2: the second term times
//          b, and db = -beta k * (W~^T g));
//   G <- G - beta g kk^T  (the adjoint of W~), then through the decay:
//   dalpha_t = <G, W_{t-1}> and G <- alpha G  (scalar decay), or per key
//   channel dalpha_t[j] = sum_i G_ij W_{t-1,ij} and G <- G diag(alpha).
// After token 0, dstate_in = G.
//
// Schedule.  One workgroup per (b, h, ROWS rows of W), as the token-recurrent
// forward (rows of W are independent in the forward, and in the adjoint
// every row-local quantity stays row-local): TPR lanes per row, each lane
// CPT = dk / TPR columns (column lr + TPR m).
//   Phase 1: the forward recurrence, writing W before every chunk of CB
//            tokens to the workspace (each lane its own columns).
//   Phase 2: the chunks in reverse.  Each lane reloads the chunk's
//            checkpoint (the values it wrote itself), recomputes the states
//            before each of the chunk's tokens into registers, and carries
//            G back token by token.
// dv, dw and dstate_in are row-local and written directly.  dq, dk, dbeta,
// dalpha and db sum over all dv rows: each wave sums its rows with lane
// shuffles, the workgroup's waves through LDS every HB tokens, and the
// workgroups of a head (dv / ROWS of them) add into zeroed fp32 outputs
// with vector atomics, so those sums are not bitwise reproducible run to run
// (their order of addition varies); every other output is.
#include <algorithm>

#include "device_common.h"
#include "lam_internal.h"

namespace lam {
namespace {

constexpr int kBw = 256;  // threads per workgroup
constexpr int CB = 16;    // tokens per checkpoint chunk
constexpr int HB = 8;     // tokens per flush of the cross-row sums

template <int DK>
struct BwShape {
    static constexpr int TPR = DK >= 64 ? 16 : 8;  // lanes per row
    static constexpr int CPT = DK / TPR;           // columns per lane
    static constexpr int ROWS = kBw / TPR;         // rows per workgroup
};

// Sum over the rows of a wave: lanes lr, lr + TPR, lr + 2 TPR, ...  The
// partner across 16 and 32 lanes comes from gfx950's row-swap moves (with a
// value swapped against itself, the two results are the two halves of each
// pair, so their sum is the pair's sum in every lane); the partner across 8
// lanes is a rotation by 8 inside each 16-lane row.  All VALU, no LDS.
__device__ __forceinline__ float swap_sum16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_sum32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Two row sums for the price of one: with a and b swapped against each other
// across 16 lanes, the pair sums of a land in 16-lane rows 0 and 2 and those
// of b in rows 1 and 3; one 32-lane swap then completes both.  Returns a's
// total in lanes 0-15 (and 32-47) and b's in lanes 16-31 (and 48-63).
template <int TPR>
__device__ __forceinline__ float wave_rows_sum2(float a, float b) {
    if constexpr (TPR <= 8) {  // memory rows of 8 lanes: first the partner 8 lanes on (row_ror:8)
        a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x128, 0xf, 0xf, false));
        b += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(b), 0x128, 0xf, 0xf, false));
    }
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return swap_sum32(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

template <int VARIANT, typename IO, int DK>
__global__ __launch_bounds__(kBw) void delta_backward_kernel(DeltaBwdArgs g) {
    using Sh = BwShape<DK>;
    constexpr int TPR = Sh::TPR, CPT = Sh::CPT, ROWS = Sh::ROWS;
    constexpr bool kChan = VARIANT == kKimiDelta;
    constexpr bool kScalar = VARIANT == kGatedDeltaNet || VARIANT == kGatedDeltaNet2;
    constexpr bool kGates2 = VARIANT == kGatedDeltaNet2;
    constexpr bool kX = kChan || kGates2;  // a per-channel tile: decays (Kimi Delta) or erase gates
    constexpr int KSL = CB * DK / kBw, VSL = CB * ROWS / kBw;
    static_assert(CB * DK % kBw == 0 && CB * ROWS % kBw == 0, "tile slots");
    const DeltaArgs &a = g.f;

    const int T = static_cast<int>(a.T), H = static_cast<int>(a.H), dv = a.dv;
    const int slices = dv / ROWS;
    int head, slice;
    xcd_group_map(blockIdx.x, static_cast<int>(a.B * a.H), slices, head, slice);
    const int b = head / H, h = head % H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = tid % TPR, rl = tid / TPR, row = slice * ROWS + rl;
    const int nch = (T + CB - 1) / CB;

    __shared__ float sq[CB][DK], sk[CB][DK], sx[kX ? CB : 1][kX ? DK : 1];
    __shared__ float sv[CB][ROWS], sw[kGates2 ? CB : 1][kGates2 ? ROWS : 1], sdy[CB][ROWS];
    __shared__ float sbeta[CB], salpha[CB];
    __shared__ float rq[HB][4][DK], rk[HB][4][DK], rx[kX ? HB : 1][4][kX ? DK : 1], rs[HB][4][2];

    // ---- chunk staging: registers (loaded one chunk ahead) -> LDS
    float fq[KSL], fk[KSL], fx[kX ? KSL : 1], fv[VSL], fw[kGates2 ? VSL : 1], fdy[VSL];
    float fbeta = 0.f, falpha = 1.f;
    auto tokidx = [&](int t) { return (static_cast<int64_t>(b) * T + t) * H + h; };
    auto fetch = [&](int c, bool rev) {  // rev: also the queries and dout
        const int t0 = c * CB;
#pragma unroll
        for (int s = 0; s < KSL; ++s) {
            const int e = tid + kBw * s, t = e / DK, j = e % DK, tt = t0 + t;
            const bool ok = tt < T;
            const int64_t gi = tokidx(min(tt, T - 1)) * DK + j;
            fq[s] = ok && rev ? IO::ld(a.q, gi) : 0.f;
            fk[s] = ok ? IO::ld(a.k, gi) : 0.f;
            if constexpr (kChan) fx[s] = ok ? IO::ld(a.alpha, gi) : 1.f;
            if constexpr (kGates2) fx[s] = ok ? IO::ld(a.erase_b, gi) : 0.f;
        }
#pragma unroll
        for (int s = 0; s < VSL; ++s) {
            const int e = tid + kBw * s, t = e / ROWS, i = e % ROWS, tt = t0 + t;
            const bool ok = tt < T;
            const int64_t gi = tokidx(min(tt, T - 1)) * dv + slice * ROWS + i;
            fv[s] = ok ? IO::ld(a.v, gi) : 0.f;
            if constexpr (kGates2) fw[s] = ok ? IO::ld(a.write_w, gi) : 0.f;
            fdy[s] = ok && rev ? IO::ld(g.dout, gi) : 0.f;
        }
        if (tid < CB) {
            const int tt = t0 + tid;
            const bool ok = tt < T;
            fbeta = ok ? IO::ld(a.beta, tokidx(min(tt, T - 1))) : 0.f;
            if constexpr (kScalar) falpha = ok ? IO::ld(a.alpha, tokidx(min(tt, T - 1))) : 1.f;
        }
    };
    auto commit = [&]() {
#pragma unroll
        for (int s = 0; s < KSL; ++s) {
            const int e = tid + kBw * s, t = e / DK, j = e % DK;
            sq[t][j] = fq[s];
            sk[t][j] = fk[s];
            if constexpr (kX) sx[t][j] = fx[s];
        }
#pragma unroll
        for (int s = 0; s < VSL; ++s) {
            const int e = tid + kBw * s, t = e / ROWS, i = e % ROWS;
            sv[t][i] = fv[s];
            if constexpr (kGates2) sw[t][i] = fw[s];
            sdy[t][i] = fdy[s];
        }
        if (tid < CB) {
            sbeta[tid] = fbeta;
            salpha[tid] = falpha;
        }
    };
    // decay of column m of token t, and the read key
    auto decay = [&](int t, int m) {
        if constexpr (kChan) return sx[t][lr + TPR * m];
        if constexpr (kScalar) return salpha[t];
        return 1.f;
    };
    auto rkey = [&](int t, int m) {
        const float kj = sk[t][lr + TPR * m];
        if constexpr (kGates2) return sx[t][lr + TPR * m] * kj;
        return kj;
    };
    // one forward token on this lane's columns of its row (padding tokens --
    // k = 0, beta = 0, decay 1 -- leave W unchanged)
    auto fwd = [&](float (&W)[CPT], int t) {
        float p = 0.f;
#pragma unroll
        for (int m = 0; m < CPT; ++m) {
            W[m] *= decay(t, m);
            p = fmaf(W[m], rkey(t, m), p);
        }
        p = group_sum<TPR>(p);
        float z = sv[t][rl];
        if constexpr (kGates2) z *= sw[t][rl];
        const float br = sbeta[t] * (z - p);
#pragma unroll
        for (int m = 0; m < CPT; ++m) W[m] = fmaf(br, sk[t][lr + TPR * m], W[m]);
    };

    const int64_t sbase = (static_cast<int64_t>(head) * dv + row) * DK;
    float *ck = g.ckpt + static_cast<int64_t>(head) * nch * dv * DK;  // [chunk][dv][dk] of this head

    // ---------------------------- phase 1: forward ----------------------------
    float W[CPT];
#pragma unroll
    for (int m = 0; m < CPT; ++m) W[m] = a.state_in ? a.state_in[sbase + lr + TPR * m] : 0.f;
    if (nch > 0) fetch(0, false);
    for (int c = 0; c < nch; ++c) {
        __syncthreads();  // the previous chunk's tiles consumed
        commit();
        __syncthreads();
        if (c + 1 < nch) fetch(c + 1, false);
        float *cp = ck + (static_cast<int64_t>(c) * dv + row) * DK;
#pragma unroll
        for (int m = 0; m < CPT; ++m) cp[lr + TPR * m] = W[m];
        for (int t = 0; t < CB; ++t) fwd(W, t);
    }

    // ---------------------------- phase 2: reverse ----------------------------
    float G[CPT];
#pragma unroll
    for (int m = 0; m < CPT; ++m) G[m] = g.dstate_out ? g.dstate_out[sbase + lr + TPR * m] : 0.f;
    if (nch > 0) fetch(nch - 1, true);
    for (int c = nch - 1; c >= 0; --c) {
        __syncthreads();
        commit();
        __syncthreads();
        if (c > 0) fetch(c - 1, true);
        // the states before each token of the chunk, from its checkpoint
        // (written by this lane in phase 1)
        float Ws[CB][CPT];
        const float *cp = ck + (static_cast<int64_t>(c) * dv + row) * DK;
#pragma unroll
        for (int m = 0; m < CPT; ++m) Ws[0][m] = cp[lr + TPR * m];
#pragma unroll
        for (int t = 0; t + 1 < CB; ++t) {
#pragma unroll
            for (int m = 0; m < CPT; ++m) Ws[t + 1][m] = Ws[t][m];
            fwd(Ws[t + 1], t);
        }
        const int t0 = c * CB;
#pragma unroll
        for (int hh = 1; hh >= 0; --hh) {
#pragma unroll
            for (int tt = HB - 1; tt >= 0; --tt) {
                const int t = hh * HB + tt;
                const float be = sbeta[t];
                // W~ and the residual, recomputed from W_{t-1}
                float wt[CPT], kk[CPT], dcy[CPT];
                float p = 0.f;
#pragma unroll
                for (int m = 0; m < CPT; ++m) {
                    dcy[m] = decay(t, m);
                    wt[m] = Ws[t][m] * dcy[m];
                    kk[m] = rkey(t, m);
                    p = fmaf(wt[m], kk[m], p);
                }
                p = group_sum<TPR>(p);
                float z = sv[t][rl];
                if constexpr (kGates2) z *= sw[t][rl];
                const float r = z - p, br = be * r;
                const float dyi = sdy[t][rl];
                // the read: G += dout q^T, dq = W_t^T dout with W_t = W~ + beta r k^T
                float pq[CPT], gk = 0.f;
#pragma unroll
                for (int m = 0; m < CPT; ++m) {
                    const int j = lr + TPR * m;
                    const float kj = sk[t][j];
                    G[m] = fmaf(dyi, sq[t][j], G[m]);
                    pq[m] = fmaf(br, kj, wt[m]) * dyi;
                    gk = fmaf(G[m], kj, gk);
                }
                gk = group_sum<TPR>(gk);
                // the write
                const float dz = be * gk, nb = -be * gk;
                if (lr == 0 && t0 + t < T) {
                    const int64_t vi = tokidx(t0 + t) * dv + row;
                    if constexpr (kGates2) {
                        g.dv[vi] = sw[t][rl] * dz;
                        g.dwrite_w[vi] = sv[t][rl] * dz;
                    } else {
                        g.dv[vi] = dz;
                    }
                }
                float pk[CPT], px[kX ? CPT : 1];
#pragma unroll
                for (int m = 0; m < CPT; ++m) {
                    const int j = lr + TPR * m;
                    const float tw = nb * wt[m];  // -beta g_i W~_ij
                    if constexpr (kGates2) {
                        pk[m] = fmaf(be * r, G[m], sx[t][j] * tw);
                        px[m] = sk[t][j] * tw;
                    } else {
                        pk[m] = fmaf(be * r, G[m], tw);
                    }
                    G[m] = fmaf(nb, kk[m], G[m]);  // the adjoint of W~
                }
                // the decay
                float da = 0.f;
#pragma unroll
                for (int m = 0; m < CPT; ++m) {
                    if constexpr (kScalar) da = fmaf(G[m], Ws[t][m], da);
                    if constexpr (kChan) px[m] = G[m] * Ws[t][m];
                    G[m] *= dcy[m];
                }
                if constexpr (kScalar) da = group_sum<TPR>(da);
                // this wave's rows summed in pairs (dq with dk, neighbouring
                // columns of the third gradient, dbeta with dalpha), into the
                // token's LDS slot: first of each pair from lanes 0 .. TPR-1,
                // second from lanes 16 .. 16+TPR-1
                float zqk[CPT], zx[kX ? CPT / 2 : 1];
#pragma unroll
                for (int m = 0; m < CPT; ++m) zqk[m] = wave_rows_sum2<TPR>(pq[m], pk[m]);
                if constexpr (kX) {
#pragma unroll
                    for (int m = 0; m < CPT / 2; ++m) zx[m] = wave_rows_sum2<TPR>(px[2 * m], px[2 * m + 1]);
                }
                const float zs = wave_rows_sum2<TPR>(r * gk, kScalar ? da : 0.f);
                const int half = lane >> 4;  // 0: first of the pair, 1: second
                if ((lane & 15) < TPR && lane < 32) {
#pragma unroll
                    for (int m = 0; m < CPT; ++m) (half ? rk : rq)[tt][wave][lr + TPR * m] = zqk[m];
                    if constexpr (kX) {
#pragma unroll
                        for (int m = 0; m < CPT / 2; ++m) rx[tt][wave][lr + TPR * (2 * m + half)] = zx[m];
                    }
                    if ((lane & 15) == 0) rs[tt][wave][half] = zs;
                }
            }
            // the workgroup's sums of these HB tokens, added into the outputs
            __syncthreads();
            const int tb = t0 + hh * HB, nv = max(0, min(HB, T - tb));
            for (int e = tid; e < nv * DK; e += kBw) {
                const int tt = e / DK, j = e % DK;
                const int64_t gi = tokidx(tb + tt) * DK + j;
                atomicAdd(&g.dq[gi], (rq[tt][0][j] + rq[tt][1][j]) + (rq[tt][2][j] + rq[tt][3][j]));
                atomicAdd(&g.dk[gi], (rk[tt][0][j] + rk[tt][1][j]) + (rk[tt][2][j] + rk[tt][3][j]));
                if constexpr (kX) {
                    const float sx_ = (rx[tt][0][j] + rx[tt][1][j]) + (rx[tt][2][j] + rx[tt][3][j]);
                    atomicAdd(kChan ? &g.dalpha[gi] : &g.derase_b[gi], sx_);
                }
            }
            if (tid < nv) {
                const int64_t si = tokidx(tb + tid);
                atomicAdd(&g.dbeta[si], (rs[tid][0][0] + rs[tid][1][0]) + (rs[tid][2][0] + rs[tid][3][0]));
                if constexpr (kScalar)
                    atomicAdd(&g.dalpha[si], (rs[tid][0][1] + rs[tid][1][1]) + (rs[tid][2][1] + rs[tid][3][1]));
            }
            __syncthreads();
        }
    }
    if (g.dstate_in) {
#pragma unroll
        for (int m = 0; m < CPT; ++m) g.dstate_in[sbase + lr + TPR * m] = G[m];
    }
}

// zero-fill of the outputs the workgroups add into
__global__ __launch_bounds__(256) void zero_kernel(float *p, int64_t n) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256)
        p[i] = 0.f;
}

template <int VARIANT, typename IO, int DK>
hipError_t launch3(const DeltaBwdArgs &g, hipStream_t stream) {
    const DeltaArgs &a = g.f;
    const unsigned blocks = static_cast<unsigned>(a.B * a.H * (a.dv / BwShape<DK>::ROWS));
    delta_backward_kernel<VARIANT, IO, DK><<<blocks, kBw, 0, stream>>>(g);
    return hipGetLastError();
}

template <int VARIANT, typename IO>
hipError_t launch2(const DeltaBwdArgs &g, hipStream_t stream) {
    switch (g.f.dk) {
        case 32: return launch3<VARIANT, IO, 32>(g, stream);
        case 64: return launch3<VARIANT, IO, 64>(g, stream);
        case 96: return launch3<VARIANT, IO, 96>(g, stream);
        case 128: return launch3<VARIANT, IO, 128>(g, stream);
    }
    return hipErrorInvalidValue;
}

template <typename IO>
hipError_t launch1(const DeltaBwdArgs &g, hipStream_t stream) {
    switch (g.f.variant) {
        case kDeltaNet: return launch2<kDeltaNet, IO>(g, stream);
        case kGatedDeltaNet: return launch2<kGatedDeltaNet, IO>(g, stream);
        case kKimiDelta: return launch2<kKimiDelta, IO>(g, stream);
        case kGatedDeltaNet2: return launch2<kGatedDeltaNet2, IO>(g, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t zero(float *p, int64_t n, hipStream_t stream) {
    if (!p || n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    zero_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(p, n);
    return hipGetLastError();
}

}  // namespace

bool delta_backward_workspace(const DeltaArgs &a, size_t *bytes) {
    const int rows = a.dk >= 64 ? 16 : 32;
    if (a.dv % rows != 0) return false;
    const int64_t nch = (a.T + CB - 1) / CB;
    *bytes = kStatusBytes + static_cast<size_t>(a.B * a.H * nch) * a.dv * a.dk * sizeof(float);
    return true;
}

hipError_t launch_delta_backward(const DeltaBwdArgs &g, hipStream_t stream) {
    const DeltaArgs &a = g.f;
    const int64_t n = a.B * a.T * a.H;
    hipError_t e;
    // the status word (no bounded waits here: it stays 0)
    if ((e = zero(static_cast<float *>(a.ws), 1, stream)) != hipSuccess) return e;
    if ((e = zero(g.dq, n * a.dk, stream)) != hipSuccess) return e;
    if ((e = zero(g.dk, n * a.dk, stream)) != hipSuccess) return e;
    if ((e = zero(g.dbeta, n, stream)) != hipSuccess) return e;
    if (a.variant != kDeltaNet && (e = zero(g.dalpha, a.variant == kKimiDelta ? n * a.dk : n, stream)) != hipSuccess)
        return e;
    if (a.variant == kGatedDeltaNet2 && (e = zero(g.derase_b, n * a.dk, stream)) != hipSuccess) return e;
    return a.dtype == kBF16 ? launch1<IoBF16>(g, stream) : launch1<IoF32>(g, stream);
}

}  // namespace lam
