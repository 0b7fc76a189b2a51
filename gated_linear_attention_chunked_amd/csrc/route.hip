// route.hip -- the cross-layer routing epilogue on gfx950 matrix cores:
// h <- h + s P^T ("Mechanisms, trade-offs and cross-layer routing of
// linear-attention architectures", "Methodology" and "Technical details": a
// zero-initialised projection P maps each token's routing signal s -- the
// delta-rule residual or the write value of every head -- to the model width,
// and epsilon = P s is added to the residual stream h).
//
// A plain contraction over the signal width N with both operands N-major
// (s is [M, N], P is [D, N]), so each 16-byte piece of a row is a run of
// eight (bf16) or four (fp32) reduction indices: exactly an MFMA operand
// fragment.  The add is fused into the epilogue, so h is read once and
// written once.
//
// Schedule: one workgroup of 4 waves per 128-token x 128-column tile of h,
// two workgroups per compute unit (74 KB of LDS each), so one's load waits
// are covered by the other's products.  Per step of BK reduction indices the
// workgroup stages its s rows and P rows into LDS (rows padded by 16 bytes,
// so the 16 lanes reading one fragment hit distinct banks) while it
// multiplies the previous step's tiles; waves own 64 x 64 sub-tiles (16
// accumulator tiles of 16 x 16).  The product is formed
// transposed, C^T = P s^T, so a lane's accumulator holds four consecutive
// columns of h for one token: the epilogue reads, adds and writes 8 (bf16) or
// 16 (fp32) contiguous bytes per lane and tile.  The eight column tiles of a
// token tile run on one XCD (its s rows are fetched from HBM once); P is
// small and stays in every XCD's L2.
#include <type_traits>

#include "chunk_common.h"
#include "lam_internal.h"

namespace lam {
namespace {

constexpr int RBM = 128;    // tokens per workgroup tile
constexpr int RBD = 128;    // columns of h per workgroup tile
constexpr int RNT = 256;    // threads
constexpr int PIECES = 8;   // 16-byte pieces per staged row (BK elements)

template <typename IO>
struct RouteTraits;
template <>
struct RouteTraits<IoBF16> {
    using E = __bf16;
    static constexpr int EPP = 8;  // elements per 16-byte piece
};
template <>
struct RouteTraits<IoF32> {
    using E = float;
    static constexpr int EPP = 4;
};

template <typename IO>
struct RouteLds {
    using E = typename RouteTraits<IO>::E;
    static constexpr int BK = PIECES * RouteTraits<IO>::EPP;   // reduction indices per step
    static constexpr int RS = BK + RouteTraits<IO>::EPP;       // padded row stride (elements)
    alignas(16) E a[2][RBM * RS];   // s rows
    alignas(16) E b[2][RBD * RS];   // P rows
};

typedef float f32x4v __attribute__((ext_vector_type(4)));

template <typename IO>
__global__ __launch_bounds__(RNT) void route_kernel(int64_t M, int D, int N, const void *__restrict__ sv,
                                                    const void *__restrict__ pv, void *__restrict__ hv) {
    using Tr = RouteTraits<IO>;
    using E = typename Tr::E;
    using L = RouteLds<IO>;
    constexpr int BK = L::BK, RS = L::RS, EPP = Tr::EPP;
    constexpr bool kBf16 = std::is_same<IO, IoBF16>::value;
    __shared__ L s;

    const int mtiles = static_cast<int>((M + RBM - 1) / RBM), dtiles = (D + RBD - 1) / RBD;
    int mt, dt;
    xcd_group_map(blockIdx.x, mtiles, dtiles, mt, dt);
    const int64_t m0 = static_cast<int64_t>(mt) * RBM;
    const int d0 = dt * RBD;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wd = wave & 1;   // sub-tile: tokens 64 wm .., columns 64 wd ..
    const int lg = lane >> 4, lc = lane & 15;
    const E *S = static_cast<const E *>(sv);
    const E *P = static_cast<const E *>(pv);

    // staging: piece i of the thread covers row (tid + RNT i) / 8, piece (tid % 8)
    constexpr int NA = RBM * PIECES / RNT, NB = RBD * PIECES / RNT;
    const int prow = tid / PIECES, pc = tid % PIECES;
    // Loads are unconditional (rows and reduction indices clamped into the
    // operands) so they stay in flight through the products; pieces outside
    // the operands are zeroed at commit.
    uint4 ra[NA], rb[NB];
    uint32_t okm = 0u;  // bit i: A piece i inside; bit NA + i: B piece i inside
    const E *arow[NA];
    const E *brow[NB];
#pragma unroll
    for (int i = 0; i < NA; ++i) arow[i] = S + min(m0 + prow + (RNT / PIECES) * i, M - 1) * N;
#pragma unroll
    for (int i = 0; i < NB; ++i) brow[i] = P + static_cast<int64_t>(min(d0 + prow + (RNT / PIECES) * i, D - 1)) * N;
    auto fetch = [&](int k0) {
        const int kk = k0 + pc * EPP;
        const bool kin = kk < N;
        const int kc = min(kk, N - EPP);
        okm = 0u;
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            okm |= (kin && m0 + prow + (RNT / PIECES) * i < M ? 1u : 0u) << i;
            ra[i] = *reinterpret_cast<const uint4 *>(arow[i] + kc);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            okm |= (kin && d0 + prow + (RNT / PIECES) * i < D ? 1u : 0u) << (NA + i);
            rb[i] = *reinterpret_cast<const uint4 *>(brow[i] + kc);
        }
    };
    auto mask = [](uint4 x, uint32_t m) { return make_uint4(x.x & m, x.y & m, x.z & m, x.w & m); };
    auto commit = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NA; ++i)
            *reinterpret_cast<uint4 *>(&s.a[buf][(prow + (RNT / PIECES) * i) * RS + pc * EPP]) =
                mask(ra[i], 0u - ((okm >> i) & 1u));
#pragma unroll
        for (int i = 0; i < NB; ++i)
            *reinterpret_cast<uint4 *>(&s.b[buf][(prow + (RNT / PIECES) * i) * RS + pc * EPP]) =
                mask(rb[i], 0u - ((okm >> (NA + i)) & 1u));
    };

    // acc[j][i]: C^T tile of columns 64 wd + 16 j .. (rows of the transposed
    // product) by tokens 64 wm + 16 i ..; lane (lg, lc) holds columns
    // 4 lg .. 4 lg + 3 of token lc
    constexpr int MI = 4;  // token tiles per wave
    f32x4 acc[4][MI];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < MI; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto multiply = [&](int buf) {
        const E *A = s.a[buf] + (64 * wm) * RS;
        const E *B = s.b[buf] + (64 * wd) * RS;
        if constexpr (kBf16) {
#pragma unroll
            for (int k = 0; k < BK; k += 32) {
                bf16x8 pf[4], sf[MI];
#pragma unroll
                for (int j = 0; j < 4; ++j) pf[j] = row_frag2(B, RS, 16 * j, k, lane);
#pragma unroll
                for (int i = 0; i < MI; ++i) sf[i] = row_frag2(A, RS, 16 * i, k, lane);
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int i = 0; i < MI; ++i) acc[j][i] = mfma32(pf[j], sf[i], acc[j][i]);
            }
        } else {
            // four reduction indices per lane and read (16 bytes); the four
            // products take element r of every lane's run, so A and B agree
            // on which index each lane supplies
#pragma unroll
            for (int k = 0; k < BK; k += 16) {
                f32x4v pf[4], sf[MI];
                typedef __attribute__((address_space(3))) const f32x4v lds_f4;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    pf[j] = *reinterpret_cast<lds_f4 *>((__attribute__((address_space(3))) const void *)(
                        B + (16 * j + lc) * RS + k + 4 * lg));
#pragma unroll
                for (int i = 0; i < MI; ++i)
                    sf[i] = *reinterpret_cast<lds_f4 *>((__attribute__((address_space(3))) const void *)(
                        A + (16 * i + lc) * RS + k + 4 * lg));
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int i = 0; i < MI; ++i)
                            acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x4f32(pf[j][r], sf[i][r], acc[j][i], 0, 0, 0);
            }
        }
    };

    const int nk = (N + BK - 1) / BK;
    fetch(0);
    commit(0);
    __syncthreads();
    for (int kb = 0; kb < nk; ++kb) {
        const int buf = kb & 1;
        if (kb + 1 < nk) fetch((kb + 1) * BK);  // in flight during the products
        multiply(buf);
        if (kb + 1 < nk) commit(buf ^ 1);       // the other buffer: last read before the previous barrier
        __syncthreads();
    }

    // epilogue: h[token][4 columns] += acc, read and written once.  The h
    // reads of a half tile are all issued before any is used (clamped into
    // h, so unconditional), then added and stored where they fall inside.
    using H4 = std::conditional_t<kBf16, bf16x4, float4>;
    H4 *hp = static_cast<H4 *>(hv);
#pragma unroll
    for (int half = 0; half < MI / 4; ++half) {
        H4 hx[4][4];
        int64_t off[4][4];
        bool in[4][4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int i = 4 * half + ii;
            const int64_t m = m0 + 64 * wm + 16 * i + lc;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d = d0 + 64 * wd + 16 * j + 4 * lg;
                in[ii][j] = m < M && d < D;
                off[ii][j] = (min(m, M - 1) * D + min(d, D - 4)) / 4;
                hx[ii][j] = hp[off[ii][j]];
            }
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 a4 = acc[j][4 * half + ii];
                if constexpr (kBf16) {
                    const f32x4 x = __builtin_convertvector(hx[ii][j], f32x4) + a4;
                    if (in[ii][j]) hp[off[ii][j]] = bf4(x);
                } else {
                    const float4 x = hx[ii][j];
                    if (in[ii][j]) hp[off[ii][j]] = make_float4(x.x + a4[0], x.y + a4[1], x.z + a4[2], x.w + a4[3]);
                }
            }
    }
}

}  // namespace

bool route_supported(int64_t D, int64_t N) { return D > 0 && N > 0 && D % 16 == 0 && N % 32 == 0; }

hipError_t launch_route(int dtype, int64_t M, int64_t D, int64_t N, const void *s, const void *P, void *h,
                        hipStream_t stream) {
    if (M == 0) return hipSuccess;
    const int64_t blocks = ((M + RBM - 1) / RBM) * ((D + RBD - 1) / RBD);
    if (dtype == kBF16)
        route_kernel<IoBF16><<<static_cast<unsigned>(blocks), RNT, 0, stream>>>(M, static_cast<int>(D),
                                                                                static_cast<int>(N), s, P, h);
    else
        route_kernel<IoF32><<<static_cast<unsigned>(blocks), RNT, 0, stream>>>(M, static_cast<int>(D),
                                                                               static_cast<int>(N), s, P, h);
    return hipGetLastError();
}

}  // namespace lam
