// loglin_recurrent.hip -- log-linear (Fenwick-tree) readout of the delta-rule
// family on gfx950, token by token, and its adaptive level weights.
//
// "Technical summary: adaptive memory decay for log-linear attention",
// "Problem definition": the memory is organised as a Fenwick-tree hierarchy
// of O(log T) levels and each step's output is a lambda^(l)_t-weighted sum of
// the levels' reads; "Methodology" (LambdaMLPSoftplus): lambda_t =
// softplus((d_t W1) W2 + b) per token, head and level; "Complexity
// preservation": O(log T) decoding memory.
//
// Readings.  For the query at absolute position t, token t is level 0 and an
// earlier token s is level msb(t xor s) + 1 (the lowbit segments of [0, t)).
// Every level's memory takes the variant's transition each step (decay, then
// the delta-rule erase along e with that level's own prediction), only level
// 0 receives the new write beta z k^T, and at position t >= 1 levels
// 0 .. ctz(t) merge into level ctz(t) + 1.  The levels sum to exactly the
// plain scan's memory, so lambda = 1 reproduces the plain scan.
//
// Schedule.  As the plain token-recurrent scan: one workgroup per (b, h,
// ROWS rows of the memory), TPR lanes per row, every level's row slice in
// registers (LMAX levels x CPT columns per lane), tokens staged through LDS
// in tiles of TT.  Per token and occupied level: decay, prediction (one
// lane-group sum), erase; then the write into level 0; then one read, the
// levels folded column by column with their lambdas before a single
// lane-group sum.  Which levels hold anything is a uniform bit mask: for
// Kimi Delta and Gated DeltaNet-2 an empty level (on average about half)
// costs one scalar branch; DeltaNet and Gated DeltaNet run every level's
// transition without branches (an empty level stays zero), which lets the
// levels' independent chains interleave.
#include "device_common.h"
#include "lam_internal.h"

namespace lam {
namespace {

constexpr int kLThreads = 256;
typedef float f32x4v __attribute__((ext_vector_type(4)));
constexpr int LTT = 16;  // tokens per LDS tile

template <int DK>
struct LlShape {
    static constexpr int TPR = DK >= 96 ? 16 : 8;
    static constexpr int CPT = DK / TPR;
    static constexpr int ROWS = kLThreads / TPR;
};

template <int VARIANT, typename IO, int DK, int LMAX>
__global__ __launch_bounds__(kLThreads) void loglin_recurrent_kernel(LogLinArgs g) {
    using Sh = LlShape<DK>;
    constexpr int TPR = Sh::TPR, CPT = Sh::CPT, ROWS = Sh::ROWS;
    constexpr bool kChanDecay = VARIANT == kKimiDelta;
    constexpr bool kScalarDecay = VARIANT == kGatedDeltaNet || VARIANT == kGatedDeltaNet2;
    constexpr bool kGates2 = VARIANT == kGatedDeltaNet2;
    constexpr bool kAllLevels = !kChanDecay && !kGates2;
    const DeltaArgs &a = g.f;

    const int T = static_cast<int>(a.T), H = static_cast<int>(a.H), dv = a.dv, nL = g.nL;
    const int slices = dv / ROWS;
    int head, slice;
    xcd_group_map(blockIdx.x, static_cast<int>(a.B * a.H), slices, head, slice);
    const int b = head / H, h = head % H;
    const int tid = threadIdx.x;
    const int lr = tid % TPR, rl = tid / TPR, row = slice * ROWS + rl;

    __shared__ float sq[LTT][DK], sk[LTT][DK];
    __shared__ float sv[LTT][ROWS];
    __shared__ float sbeta[LTT], salpha[LTT];
    __shared__ float sdec[kChanDecay ? LTT : 1][kChanDecay ? DK : 1];
    __shared__ float serase[kGates2 ? LTT : 1][kGates2 ? DK : 1];
    __shared__ float swrite[kGates2 ? LTT : 1][kGates2 ? ROWS : 1];
    __shared__ float slam[LTT][LMAX];
    __shared__ float sy[LTT][ROWS];

    // ---- every level's row slice in registers; levels >= nL stay empty
    float S[LMAX][CPT];
    const int64_t lsz = static_cast<int64_t>(dv) * DK;
    const int64_t sbase = (static_cast<int64_t>(b) * H + h) * nL * lsz + static_cast<int64_t>(row) * DK;
#pragma unroll
    for (int l = 0; l < LMAX; ++l)
#pragma unroll
        for (int m = 0; m < CPT; ++m)
            S[l][m] = (a.state_in && l < nL) ? a.state_in[sbase + l * lsz + lr + TPR * m] : 0.f;
    // levels that may hold anything (uniform): all given ones, if a state came in
    unsigned occ = a.state_in ? (nL >= 32 ? ~0u : ((1u << nL) - 1u)) : 0u;

    // ---- tile staging (as the plain recurrent scan, plus the level weights)
    constexpr int KSLOTS = (LTT * DK + kLThreads - 1) / kLThreads;
    constexpr int VSLOTS = (LTT * ROWS + kLThreads - 1) / kLThreads;
    constexpr int LSLOTS = (LTT * LMAX + kLThreads - 1) / kLThreads;
    float rq[KSLOTS], rk[KSLOTS], rdec[kChanDecay ? KSLOTS : 1], rer[kGates2 ? KSLOTS : 1];
    float rv[VSLOTS], rw[kGates2 ? VSLOTS : 1], rlam[LSLOTS];
    float rbeta = 0.f, ralpha = 1.f;
    auto tokidx = [&](int tt) { return (static_cast<int64_t>(b) * T + tt) * H + h; };
    auto fetch = [&](int t0) {
#pragma unroll
        for (int s = 0; s < KSLOTS; ++s) {
            const int e = tid + s * kLThreads, t = e / DK, j = e % DK, tt = t0 + t;
            const bool ok = e < LTT * DK && tt < T;
            const int64_t gi = tokidx(min(tt, T - 1)) * DK + j;
            rq[s] = ok ? IO::ld(a.q, gi) : 0.f;
            rk[s] = ok ? IO::ld(a.k, gi) : 0.f;
            if constexpr (kChanDecay) rdec[s] = ok ? IO::ld(a.alpha, gi) : 1.f;
            if constexpr (kGates2) rer[s] = ok ? IO::ld(a.erase_b, gi) : 0.f;
        }
#pragma unroll
        for (int s = 0; s < VSLOTS; ++s) {
            const int e = tid + s * kLThreads, t = e / ROWS, i = e % ROWS, tt = t0 + t;
            const bool ok = e < LTT * ROWS && tt < T;
            const int64_t gi = tokidx(min(tt, T - 1)) * dv + slice * ROWS + i;
            rv[s] = ok ? IO::ld(a.v, gi) : 0.f;
            if constexpr (kGates2) rw[s] = ok ? IO::ld(a.write_w, gi) : 0.f;
        }
#pragma unroll
        for (int s = 0; s < LSLOTS; ++s) {
            const int e = tid + s * kLThreads, t = e / LMAX, l = e % LMAX, tt = t0 + t;
            const bool ok = e < LTT * LMAX && tt < T && l < nL;
            rlam[s] = ok ? g.lam[tokidx(min(tt, T - 1)) * nL + l] : 0.f;
        }
        if (tid < LTT) {
            const int tt = t0 + tid;
            const bool ok = tt < T;
            const int64_t gi = tokidx(min(tt, T - 1));
            rbeta = ok ? IO::ld(a.beta, gi) : 0.f;
            if constexpr (kScalarDecay) ralpha = ok ? IO::ld(a.alpha, gi) : 1.f;
        }
    };
    auto commit = [&]() {
#pragma unroll
        for (int s = 0; s < KSLOTS; ++s) {
            const int e = tid + s * kLThreads;
            if (e < LTT * DK) {
                const int t = e / DK, j = e % DK;
                sq[t][j] = rq[s];
                sk[t][j] = rk[s];
                if constexpr (kChanDecay) sdec[t][j] = rdec[s];
                if constexpr (kGates2) serase[t][j] = rer[s];
            }
        }
#pragma unroll
        for (int s = 0; s < VSLOTS; ++s) {
            const int e = tid + s * kLThreads;
            if (e < LTT * ROWS) {
                const int t = e / ROWS, i = e % ROWS;
                sv[t][i] = rv[s];
                if constexpr (kGates2) swrite[t][i] = rw[s];
            }
        }
#pragma unroll
        for (int s = 0; s < LSLOTS; ++s) {
            const int e = tid + s * kLThreads;
            if (e < LTT * LMAX) slam[e / LMAX][e % LMAX] = rlam[s];
        }
        if (tid < LTT) {
            sbeta[tid] = rbeta;
            salpha[tid] = ralpha;
        }
    };

    if (T > 0) fetch(0);
    for (int t0 = 0; t0 < T; t0 += LTT) {
        __syncthreads();  // previous tile consumed
        commit();
        __syncthreads();
        if (t0 + LTT < T) fetch(t0 + LTT);
        const int nt = min(LTT, T - t0);
        for (int t = 0; t < nt; ++t) {
            const int64_t pos = g.t0 + t0 + t;  // absolute position
            // ---- Fenwick merge: levels 0 .. p into level p + 1, p = ctz(pos)
            if (pos > 0) {
                const int p = __builtin_ctzll(static_cast<unsigned long long>(pos));
                const unsigned low = (2u << p) - 1u;  // bits 0 .. p
                if (occ & low) {
                    float acc[CPT];
#pragma unroll
                    for (int m = 0; m < CPT; ++m) acc[m] = 0.f;
#pragma unroll
                    for (int l = 0; l < LMAX; ++l) {
                        if (l <= p && ((occ >> l) & 1u)) {
#pragma unroll
                            for (int m = 0; m < CPT; ++m) {
                                acc[m] += S[l][m];
                                S[l][m] = 0.f;
                            }
                        }
                    }
#pragma unroll
                    for (int l = 1; l < LMAX; ++l) {
                        if (l == p + 1) {
#pragma unroll
                            for (int m = 0; m < CPT; ++m) S[l][m] += acc[m];
                        }
                    }
                    occ = (occ & ~low) | (1u << (p + 1));
                }
            }
            // ---- this token's operands
            float kk[CPT], ee[CPT], qq[CPT], dd[CPT];
#pragma unroll
            for (int m = 0; m < CPT; ++m) {
                const int j = lr + TPR * m;
                kk[m] = sk[t][j];
                qq[m] = sq[t][j];
                ee[m] = kGates2 ? serase[t][j] * kk[m] : kk[m];
                dd[m] = kChanDecay ? sdec[t][j] : (kScalarDecay ? salpha[t] : 1.f);
            }
            const float be = sbeta[t];
            float z = sv[t][rl];
            if constexpr (kGates2) z *= swrite[t][rl];
            // ---- transition of every occupied level: decay, then erase with its own prediction.
            // An empty level holds zeros and stays zero under the transition, so where the
            // registers allow (scalar or no decay, no erase gate) every level takes it
            // without a branch: the levels' independent chains then interleave.
            float pr[LMAX];
#pragma unroll
            for (int l = 0; l < LMAX; ++l) {
                pr[l] = 0.f;
                if (kAllLevels || ((occ >> l) & 1u)) {
#pragma unroll
                    for (int m = 0; m < CPT; ++m) {
                        S[l][m] *= dd[m];
                        pr[l] = fmaf(S[l][m], ee[m], pr[l]);
                    }
                }
            }
#pragma unroll
            for (int l = 0; l < LMAX; ++l)
                if (kAllLevels || ((occ >> l) & 1u)) pr[l] = group_sum<TPR>(pr[l]);
#pragma unroll
            for (int l = 0; l < LMAX; ++l) {
                if (kAllLevels || ((occ >> l) & 1u)) {
                    const float bp = be * pr[l];
#pragma unroll
                    for (int m = 0; m < CPT; ++m) S[l][m] = fmaf(-bp, kk[m], S[l][m]);
                }
            }
            // ---- the write goes to level 0
            const float bz = be * z;
#pragma unroll
            for (int m = 0; m < CPT; ++m) S[0][m] = fmaf(bz, kk[m], S[0][m]);
            occ |= 1u;
            // ---- read: levels folded with their weights, then one lane-group sum
            float comb[CPT];
#pragma unroll
            for (int m = 0; m < CPT; ++m) comb[m] = 0.f;
#pragma unroll
            for (int l = 0; l < LMAX; ++l) {
                if ((occ >> l) & 1u) {
                    const float wl = slam[t][l];
#pragma unroll
                    for (int m = 0; m < CPT; ++m) comb[m] = fmaf(wl, S[l][m], comb[m]);
                }
            }
            float y = 0.f;
#pragma unroll
            for (int m = 0; m < CPT; ++m) y = fmaf(comb[m], qq[m], y);
            y = group_sum<TPR>(y);
            if (lr == 0) sy[t][rl] = y;
        }
        __syncthreads();
        for (int e = tid; e < nt * ROWS; e += kLThreads) {
            const int t = e / ROWS, i = e % ROWS;
            IO::st(a.out, tokidx(t0 + t) * dv + slice * ROWS + i, sy[t][i]);
        }
    }
    if (a.state_out) {
#pragma unroll
        for (int l = 0; l < LMAX; ++l)
            if (l < nL) {
#pragma unroll
                for (int m = 0; m < CPT; ++m) a.state_out[sbase + l * lsz + lr + TPR * m] = S[l][m];
            }
    }
}

template <int VARIANT, typename IO, int LMAX>
hipError_t launch_l(const LogLinArgs &g, hipStream_t stream) {
    const DeltaArgs &a = g.f;
    auto go = [&](auto kern, int rows) -> hipError_t {
        const int64_t blocks = a.B * a.H * (a.dv / rows);
        kern<<<dim3(static_cast<unsigned>(blocks)), dim3(kLThreads), 0, stream>>>(g);
        return hipGetLastError();
    };
    switch (a.dk) {
        case 32: return go(loglin_recurrent_kernel<VARIANT, IO, 32, LMAX>, LlShape<32>::ROWS);
        case 64: return go(loglin_recurrent_kernel<VARIANT, IO, 64, LMAX>, LlShape<64>::ROWS);
        case 96: return go(loglin_recurrent_kernel<VARIANT, IO, 96, LMAX>, LlShape<96>::ROWS);
        case 128: return go(loglin_recurrent_kernel<VARIANT, IO, 128, LMAX>, LlShape<128>::ROWS);
    }
    return hipErrorInvalidValue;
}

template <int VARIANT, typename IO>
hipError_t launch_v(const LogLinArgs &g, hipStream_t stream) {
    return g.nL <= 16 ? launch_l<VARIANT, IO, 16>(g, stream) : launch_l<VARIANT, IO, kLogLinMaxLevels>(g, stream);
}

template <typename IO>
hipError_t launch_io(const LogLinArgs &g, hipStream_t stream) {
    switch (g.f.variant) {
        case kDeltaNet: return launch_v<kDeltaNet, IO>(g, stream);
        case kGatedDeltaNet: return launch_v<kGatedDeltaNet, IO>(g, stream);
        case kKimiDelta: return launch_v<kKimiDelta, IO>(g, stream);
        case kGatedDeltaNet2: return launch_v<kGatedDeltaNet2, IO>(g, stream);
    }
    return hipErrorInvalidValue;
}

// ---- adaptive level weights: one thread per (token, head) row.  NLP is
// the level count rounded up to a multiple of 4: the weights are staged
// zero-padded to it, so every loop has a constant trip count and the padded
// levels add zeros; W1 is staged transposed so both products read four
// levels' weights per (broadcast) LDS access.
constexpr int kMlpThreads = 256;

template <typename IO, int NLP>
__global__ __launch_bounds__(kMlpThreads) void loglin_lambda_kernel(int64_t M, int nL, int nh, const void *d,
                                                                    const float *W1, const float *W2,
                                                                    const float *bias, float *lam) {
    __shared__ f32x4v w1t[kLogLinMaxHidden][NLP / 4];  // w1t[j][l] = W1[l][j]
    __shared__ f32x4v w2s[kLogLinMaxHidden][NLP / 4];  // w2s[j][l] = W2[j][l]
    __shared__ float bs[NLP];
    // The workgroup's rows (inputs, then outputs) pass through LDS, so that
    // global loads and stores run over consecutive addresses.  Thread t owns
    // the nL words of row t: for odd nL the lanes' accesses to one level hit
    // distinct banks, for even nL a few share one.
    __shared__ float io[kMlpThreads * NLP];
    float *w1f = reinterpret_cast<float *>(w1t), *w2f = reinterpret_cast<float *>(w2s);
    for (int e = threadIdx.x; e < nh * NLP; e += kMlpThreads) {
        const int jj = e / NLP, l = e % NLP;
        w1f[e] = l < nL ? W1[l * nh + jj] : 0.f;
        w2f[e] = l < nL ? W2[jj * nL + l] : 0.f;
    }
    if (threadIdx.x < NLP) bs[threadIdx.x] = threadIdx.x < nL ? bias[threadIdx.x] : 0.f;
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kMlpThreads;
    const int nrows = static_cast<int>(min(static_cast<int64_t>(kMlpThreads), M - r0));
    const int ne = nrows * nL;
    for (int e = threadIdx.x; e < ne; e += kMlpThreads) io[e] = IO::ld(d, r0 * nL + e);
    __syncthreads();
    const int t = threadIdx.x;
    const bool live = t < nrows;
    float x[NLP], o[NLP];
#pragma unroll
    for (int l = 0; l < NLP; ++l) {
        x[l] = (l < nL && live) ? io[t * nL + l] : 0.f;
        o[l] = bs[l];
    }
    // h = d W1 one hidden unit at a time, folded straight into h W2
    for (int jj = 0; jj < nh; ++jj) {
        float hj = 0.f;
#pragma unroll
        for (int q = 0; q < NLP / 4; ++q) {
            const f32x4v w = w1t[jj][q];
            hj = fmaf(x[4 * q], w[0], hj);
            hj = fmaf(x[4 * q + 1], w[1], hj);
            hj = fmaf(x[4 * q + 2], w[2], hj);
            hj = fmaf(x[4 * q + 3], w[3], hj);
        }
#pragma unroll
        for (int q = 0; q < NLP / 4; ++q) {
            const f32x4v w = w2s[jj][q];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[4 * q + e] = fmaf(hj, w[e], o[4 * q + e]);
        }
    }
    // softplus(x) = max(x, 0) + log1p(exp(-|x|)), through LDS to the output
    __syncthreads();  // every row's inputs read before io is overwritten
    if (live) {
#pragma unroll
        for (int l = 0; l < NLP; ++l)
            if (l < nL) io[t * nL + l] = fmaxf(o[l], 0.f) + log1pf(expf(-fabsf(o[l])));
    }
    __syncthreads();
    for (int e = threadIdx.x; e < ne; e += kMlpThreads) lam[r0 * nL + e] = io[e];
}

template <typename IO>
hipError_t launch_lambda_io(int64_t M, int nL, int nh, const void *d, const float *W1, const float *W2,
                            const float *b, float *lam, hipStream_t stream) {
    const unsigned blocks = static_cast<unsigned>((M + kMlpThreads - 1) / kMlpThreads);
    switch ((nL + 3) / 4) {
        case 1: loglin_lambda_kernel<IO, 4><<<blocks, kMlpThreads, 0, stream>>>(M, nL, nh, d, W1, W2, b, lam); break;
        case 2: loglin_lambda_kernel<IO, 8><<<blocks, kMlpThreads, 0, stream>>>(M, nL, nh, d, W1, W2, b, lam); break;
        case 3: loglin_lambda_kernel<IO, 12><<<blocks, kMlpThreads, 0, stream>>>(M, nL, nh, d, W1, W2, b, lam); break;
        case 4: loglin_lambda_kernel<IO, 16><<<blocks, kMlpThreads, 0, stream>>>(M, nL, nh, d, W1, W2, b, lam); break;
        case 5: loglin_lambda_kernel<IO, 20><<<blocks, kMlpThreads, 0, stream>>>(M, nL, nh, d, W1, W2, b, lam); break;
        case 6: loglin_lambda_kernel<IO, 24><<<blocks, kMlpThreads, 0, stream>>>(M, nL, nh, d, W1, W2, b, lam); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool loglin_supported(const DeltaArgs &a, int nL) {
    const int rows = a.dk >= 96 ? 16 : 32;
    return a.dv % rows == 0 && nL >= 1 && nL <= kLogLinMaxLevels;
}

hipError_t launch_loglin(const LogLinArgs &g, hipStream_t stream) {
    return g.f.dtype == kBF16 ? launch_io<IoBF16>(g, stream) : launch_io<IoF32>(g, stream);
}

hipError_t launch_loglin_lambda(int dtype, int64_t M, int nL, int nh, const void *d, const float *W1,
                                const float *W2, const float *b, float *lam, hipStream_t stream) {
    if (M == 0) return hipSuccess;
    return dtype == kBF16 ? launch_lambda_io<IoBF16>(M, nL, nh, d, W1, W2, b, lam, stream)
                          : launch_lambda_io<IoF32>(M, nL, nh, d, W1, W2, b, lam, stream);
}

}  // namespace lam
