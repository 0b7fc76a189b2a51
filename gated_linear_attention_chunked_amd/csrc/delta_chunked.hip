// delta_chunked.hip -- chunkwise-parallel delta-rule scan on gfx950 matrix
// cores (DeltaNet, Gated DeltaNet, Gated DeltaNet-2; bf16 streams, fp32 state).
//
// The rule ("Mechanisms, trade-offs and cross-layer routing of
// linear-attention architectures", "Technical details"): W_t = a_t W_{t-1} +
// beta_t r_t k_t^T with r_t = z_t - a_t W_{t-1} e_t and y_t = W_t q_t (e = k,
// z = v except for Gated DeltaNet-2's erase/write gates; a = 1 for DeltaNet).
//
// Chunked form (derived from that rule by unrolling it over a chunk of C
// tokens; rows = tokens, S = memory at the chunk start, g_t = sum_{j<=t}
// log a_j, gamma_t = exp(g_t), Gamma_ts = exp(g_t - g_s) for s <= t):
//   N  = strict_lower(E K^T * Gamma)
//   R  = (I + N diag(beta))^{-1} (Z - diag(gamma) E S^T)
//   Y  = diag(gamma) Q S^T + (lower(Q K^T) * Gamma) diag(beta) R
//   S' = gamma_C S + R^T diag(beta gamma_C / gamma) K
// Row t of R is token t's residual r_t, taken against the decayed memory
// (the write is beta_t r_t k_t^T): R satisfies R = Z - diag(gamma) E S^T -
// N diag(beta) R, which is the rule's residual with the chunk's earlier
// writes included.  Solving for R rather than diag(beta) R keeps beta out of
// the solve's right-hand side: the residual a caller asks for as a routing
// signal is exactly the operand the scan carries, at any beta (zero
// included), and beta enters only as a column scale of the products that
// consume R.
// Every exponent is g_t - g_s with s <= t (or g_C - g_t), so no factor exceeds
// one and strong decays underflow to zero instead of overflowing.
//
// Two kernels per call:
//   derivation: one workgroup per (sequence, head, chunk), all chunks at once.
//          It forms everything that does not depend on the state (the
//          inverses of the diagonal blocks of I + L, the off-diagonal coupling
//          blocks and the gate prefix sums) from the keys, decays and betas
//          alone, and writes it to a workspace block of 5.75 KB per chunk (in
//          the caller's workspace, after its status block).
//   scan:  one workgroup of 8 waves per (b, h, 32-wide slice of dv); rows of
//          W are independent, so slices never communicate.  Waves are split
//          into a carry, an output and a producer role; see the pipelined
//          schedule below.  The four slices of a head read the same workspace
//          blocks, so the solve's derivation is done once per head instead of
//          once per slice; the output waves form lower(Q K^T * Gamma) from
//          the staged query and key rows, which spares the derivation a read
//          of the queries.
// The state slice S^T (dk x 16 per carry wave) lives in MFMA accumulator
// layout for the whole scan.  An accumulator tile holds 4 consecutive rows per
// lane, while a B operand wants 8 consecutive reduction indices; since a
// contraction does not care how its reduction index is ordered, two stacked
// accumulator tiles serve directly as a B operand if the A operand is read
// with the same order (rows 4g..4g+3 and 16+4g..16+4g+3 of each 32-block).
// The same trick feeds R and the solve's right-hand sides to the next
// products without an LDS round trip.
#include <type_traits>

#include "chunk_common.h"
#include "lam_internal.h"

namespace lam {
namespace {

constexpr int C = 64;    // chunk length (tokens)
constexpr int BV = 32;   // dv columns per workgroup

// ===========================================================================
// With D_i = (I + N_ii diag(beta)_i)^{-1} the inverse of diagonal block i,
// G~_ij = Gamma * (E_i K_j^T) and Z = E S^T, block row i of the solve is
//     R_i = D_i Z'_i - D_i diag(gamma)_i Z_i + sum_{j<i} M_ij R_j,
//     M_ij = -D_i G~_ij diag(beta)_j                (Z' = the targets V)
// so everything but Z is state-independent: the derivation kernel forms it.
// The output's intra-chunk matrix Aqk = lower(Q K^T * Gamma) diag(beta) is
// formed by the scan's output waves from the staged query and key rows, each
// the blocks of its own token rows.
//
// Pipelined scan: 8 waves per workgroup, two per SIMD, in three roles.
//   carry  (waves 0-1, one 16-column tile each): Z = E S^T on MFMA, the
//          block solve above on 16x16x16 MFMA (a four-link chain), publish R,
//          then the state update accumulated in registers.
//   output (waves 2-3): token row tiles {0, 3} and {1, 2} for both value
//          tiles: Q S^T from the carries' bf16 states and the Aqk blocks of
//          their rows from the staged rows, then Y = diag(gamma) Q S^T + Aqk R
//          once both R are published; stores y.
//   producers (waves 4-7): stage chunk c+1 into LDS, its token rows and its
//          derived block (loads issued two chunks ahead).
// All eight waves meet at one LDS barrier per chunk; the hand-offs inside a
// chunk go through bounded LDS counters.  The chunk loop is unrolled by the
// double-buffer parity so every LDS address is a per-lane base plus a
// constant.
// ===========================================================================
constexpr int NLB = 6;     // strictly lower 16x16 blocks of a 64-row chunk
constexpr int NQB = 10;    // lower 16x16 blocks including the diagonal
constexpr int NT8 = 512;   // threads per workgroup of the scan
constexpr int NTD = 256;   // threads per workgroup of the derivation
constexpr int LTS = 20;    // column stride (floats) of the fp32 diagonal blocks

// State-independent matrices of one chunk.  The derivation kernel writes one
// block per (sequence, head, chunk); the scan copies it into LDS unchanged.
struct DerBlock {
    bf16x4 dtil[4][64];        // D_i, A-operand order
    bf16x4 mij[NLB][64];       // M_ij
    float gam[C];              // gamma_t
    float sc[C];               // beta_t gamma_C / gamma_t
    float g[C];                // log2 gamma_t
    float gb[C];               // log2 gamma_t - log2 beta_t (+inf where beta_t = 0); DeltaNet: beta_t
};
static_assert(sizeof(DerBlock) % 256 == 0, "workspace blocks stay 256-byte aligned");
constexpr int kDerPieces = static_cast<int>(sizeof(DerBlock) / 16);  // 16-byte pieces

template <int DK, bool GATES2>
struct WyLds {
    static constexpr int KS = DK + 8;
    static constexpr int VS = BV + 8;
    struct Raw {  // token rows of one chunk, double-buffered (carry/output read chunk c)
        alignas(16) __bf16 q[C * KS];
        alignas(16) __bf16 k[C * KS];
        alignas(16) __bf16 e[GATES2 ? C * KS : 8];  // erase-gated keys b * k (Gated DeltaNet-2)
        alignas(16) __bf16 v[C * VS];          // value targets of the workgroup's columns (w * v for Gated DeltaNet-2)
    };
    Raw raw[2];
    alignas(16) DerBlock der[2];
    // carry -> output
    alignas(16) bf16x4 uh[2][4][64];           // R of the current chunk, per tile
    alignas(16) bf16x4 sh[2][DK / 16][64];     // bf16 state fragments per tile
    unsigned int ucount[2];                    // R publications per tile
    unsigned int scount[2];                    // state fragments consumed per tile
};

// rows past the end become zeros (a bitwise mask keeps the registers out of
// the select-of-aggregates form that lands them in scratch)
__device__ __forceinline__ uint4 masked(uint4 x, uint32_t m) { return make_uint4(x.x & m, x.y & m, x.z & m, x.w & m); }
// elementwise product of eight bf16 pairs, rounded to bf16 (nearest even):
// widened exactly, multiplied in fp32, narrowed by the packed conversion
__device__ __forceinline__ uint4 mul8(uint4 x, uint4 y) {
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    typedef float f32x8 __attribute__((ext_vector_type(8)));
    const bf16x8 xb = __builtin_bit_cast(bf16x8, u32x4v{x.x, x.y, x.z, x.w});
    const bf16x8 yb = __builtin_bit_cast(bf16x8, u32x4v{y.x, y.y, y.z, y.w});
    const f32x8 pr = __builtin_convertvector(xb, f32x8) * __builtin_convertvector(yb, f32x8);
    const u32x4v r = __builtin_bit_cast(u32x4v, __builtin_convertvector(pr, bf16x8));
    return make_uint4(r[0], r[1], r[2], r[3]);
}

// S^T = gamma_C S^T + K^T diag(beta gamma_C / gamma) R for one 16-column tile.
template <int KT, typename Raw>
__device__ __forceinline__ void state_update(f32x4 (&St)[KT], const Raw &R, const DerBlock &D, const bf16x4 (&ub)[4],
                                             int KS, int lane) {
    const int lg = lane >> 4;
    // operand reads first, then the scaling of R while they are in flight
    bf16x8 af[2][KT];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) af[h2][kt] = col_frag(R.k, KS, 32 * h2, 16 * kt, lane);
    f32x4 us[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 sc = *reinterpret_cast<const float4 *>(&D.sc[16 * i + 4 * lg]);
        const f32x4 u = __builtin_convertvector(ub[i], f32x4);
        us[i] = u * f32x4{sc.x, sc.y, sc.z, sc.w};
    }
    const bf16x8 bW0 = cat8(bf4(us[0]), bf4(us[1])), bW1 = cat8(bf4(us[2]), bf4(us[3]));
    const float gC = D.gam[C - 1];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) St[kt] = St[kt] * gC;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) St[kt] = mfma32(af[h2][kt], h2 ? bW1 : bW0, St[kt]);
}

// E K^T tiles per derivation wave i: three each for waves 0-2, which also
// take the off-diagonal tiles of block row 3, so wave 3 only forms (3, 3).
// tmask / smask: the 16-row blocks used as rows (E) and as columns (K).
template <int I> struct RowTiles;
template <> struct RowTiles<0> {
    static constexpr int n = 3, tmask = 0x9, smask = 0x3;
    static constexpr int ti[3] = {0, 3, 3}, si[3] = {0, 0, 1};
};
template <> struct RowTiles<1> {
    static constexpr int n = 3, tmask = 0xa, smask = 0x7;
    static constexpr int ti[3] = {1, 1, 3}, si[3] = {0, 1, 2};
};
template <> struct RowTiles<2> {
    static constexpr int n = 3, tmask = 0x4, smask = 0x7;
    static constexpr int ti[3] = {2, 2, 2}, si[3] = {0, 1, 2};
};
template <> struct RowTiles<3> {
    static constexpr int n = 1, tmask = 0x8, smask = 0x8;
    static constexpr int ti[1] = {3}, si[1] = {3};
};
__device__ __forceinline__ constexpr int lower_block(int i, int j) { return i * (i - 1) / 2 + j; }  // j < i
__device__ __forceinline__ constexpr int tri_block(int i, int j) { return i * (i + 1) / 2 + j; }    // j <= i

// ============================== derivation ==============================
template <int DK, bool GATES2>
struct DeriveLds {
    static constexpr int KS = DK + 8;
    alignas(16) __bf16 k[C * KS];
    alignas(16) __bf16 e[GATES2 ? C * KS : 8];
    alignas(16) float la[C];                   // log2 of the decay (0 for padding)
    alignas(16) float beta[C];                 // beta (0 for padding)
    alignas(16) float g[C];                    // prefix sums of la
    alignas(16) float lt[4][16 * LTS];         // diagonal blocks of L, fp32, by column
    alignas(16) bf16x4 gx[3][64];              // -G~_3j (j < 3), made by waves 0 and 1 for wave 3
    alignas(16) DerBlock d;
};

// One workgroup of four waves per (sequence, head, chunk); wave i stages key
// rows [16i, 16i + 16) and then owns block row i of L: its E K^T tiles, the
// inverse of its diagonal block (fp32 forward substitution) and its M_ij.
// As the call's first kernel it also clears the status word that the scan's
// bounded waits report into.
template <int VARIANT, int DK>
__global__ __launch_bounds__(NTD) void delta_chunked_derive_kernel(DeltaArgs a, DerBlock *__restrict__ out,
                                                                   unsigned int *status) {
    constexpr bool kDecay = VARIANT != kDeltaNet;
    constexpr bool kGates2 = VARIANT == kGatedDeltaNet2;
    constexpr int KS = DK + 8;
    constexpr int KSTEP = DK / 32;
    using Lds = DeriveLds<DK, kGates2>;
    __shared__ Lds s;

    const int T = static_cast<int>(a.T), H = static_cast<int>(a.H);
    const int nchunks = (T + C - 1) / C;
    const int task = blockIdx.x;
    const int head = task / nchunks, c = task - head * nchunks;
    const int b = head / H, h = head % H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lg = lane >> 4, lc = lane & 15;
    const int t0 = c * C, last = T - 1 - t0;
    const int64_t base = (static_cast<int64_t>(b) * T + t0) * H + h;  // token index of chunk row 0
    if (task == 0 && tid == 0) *status = 0u;

    // ---- staging: a dk-wide row is DK/8 16-byte pieces, 64*8/DK rows per load
    constexpr int PPR = DK / 8, RPI = 64 / PPR, NQK = 16 / RPI;
    const uint32_t hdk = static_cast<uint32_t>(H * DK);
    const int krow = 16 * w + lane / PPR;
    const uint16_t *k0 = static_cast<const uint16_t *>(a.k) + base * DK;
    const uint16_t *b0 = static_cast<const uint16_t *>(a.erase_b) + base * DK;
    uint4 kr[NQK], br[kGates2 ? NQK : 1];
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
        const uint32_t o = static_cast<uint32_t>(min(krow + RPI * i, last)) * hdk + (lane % PPR) * 8;
        kr[i] = *reinterpret_cast<const uint4 *>(k0 + o);
        if constexpr (kGates2) br[i] = *reinterpret_cast<const uint4 *>(b0 + o);
    }
    // decay (wave 0) or beta (wave 1) of row `lane`
    uint16_t rs = 0;
    if (w == 1 || (w == 0 && kDecay)) {
        const uint16_t *gsc = static_cast<const uint16_t *>(w == 0 ? a.alpha : a.beta);
        rs = gsc[base + static_cast<int64_t>(min(lane, last)) * H];
    }
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
        const int row = krow + RPI * i;
        const uint32_t m = row <= last ? 0xffffffffu : 0u;
        *reinterpret_cast<uint4 *>(&s.k[row * KS + (lane % PPR) * 8]) = masked(kr[i], m);
        if constexpr (kGates2) *reinterpret_cast<uint4 *>(&s.e[row * KS + (lane % PPR) * 8]) = masked(mul8(kr[i], br[i]), m);
    }
    if (w == 0) s.la[lane] = (kDecay && lane <= last) ? log2_decay(bf16_bits_to_f32(rs)) : 0.f;
    if (w == 1) s.beta[lane] = lane <= last ? bf16_bits_to_f32(rs) : 0.f;
    __syncthreads();

    // ---- gate prefix sums
    DerBlock &D = s.d;
    if (w == 0) {
        const float g = wave_prefix_sum(s.la[lane]);
        const float gl = __shfl(g, 63, 64);
        s.g[lane] = g;
        D.g[lane] = g;
        D.gam[lane] = exp2_fast(g);
        D.sc[lane] = exp2_fast(gl - g) * s.beta[lane];
        // the output's column scale beta_s folded into its exponent,
        // 2^(g_t - g_s) beta_s = 2^(g_t - (g_s - log2 beta_s)); DeltaNet
        // keeps a plain factor
        D.gb[lane] = kDecay ? g - __log2f(s.beta[lane]) : s.beta[lane];
    }
    __syncthreads();

    // ---- E K^T tiles of block row I (phase 1), then the inverse of its
    // diagonal block and its M (phase 2); between them waves 0 and 1 hand
    // the row-3 Gram blocks to wave 3 through one barrier
    bf16x4 gneg[4];   // -G~_Ij in accumulator order (own block row only)
    auto gram = [&](auto ic_) {
        constexpr int I = decltype(ic_)::value;
        using Tl = RowTiles<I>;
        constexpr int NT = Tl::n;
        f32x4 acc[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < KSTEP; ++p) {
            bf16x8 kf[4], ef[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {  // key rows as columns (smask) and, unless E is
                                            // separate, as rows (tmask); E rows for Gated DeltaNet-2
                if (((kGates2 ? Tl::smask : Tl::smask | Tl::tmask) >> j) & 1)
                    kf[j] = row_frag2(s.k, KS, 16 * j, 32 * p, lane);
                if (kGates2 && ((Tl::tmask >> j) & 1)) ef[j] = row_frag2(s.e, KS, 16 * j, 32 * p, lane);
            }
#pragma unroll
            for (int j = 0; j < NT; ++j) acc[j] = mfma32(kGates2 ? ef[Tl::ti[j]] : kf[Tl::ti[j]], kf[Tl::si[j]], acc[j]);
        }
        // E K^T tiles: lane (lg, lc) holds G[t = 16ti + 4lg + r][s = 16si + lc]
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int ti = Tl::ti[j], si = Tl::si[j];
            const float4 gt4 = *reinterpret_cast<const float4 *>(&s.g[16 * ti + 4 * lg]);
            const float gt[4] = {gt4.x, gt4.y, gt4.z, gt4.w};
            const float gs = s.g[16 * si + lc];
            const float bs = s.beta[16 * si + lc];  // N diag(beta): column s's beta
            f32x4 x;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v = kDecay ? acc[j][r] * exp2_fast(fminf(gt[r] - gs, 0.f)) : acc[j][r];
                x[r] = (si < ti || lc < 4 * lg + r) ? v * bs : 0.f;
            }
            if (si == ti) {
                *reinterpret_cast<float4 *>(&s.lt[ti][lc * LTS + 4 * lg]) = make_float4(x[0], x[1], x[2], x[3]);
            } else if (ti == I) {
                gneg[si] = bf4(-x);
            } else {
                s.gx[si][lane] = bf4(-x);  // row 3 block computed for wave 3
            }
        }
    };
    if (w == 0) gram(ic<0>{});
    else if (w == 1) gram(ic<1>{});
    else if (w == 2) gram(ic<2>{});
    else gram(ic<3>{});
    __syncthreads();

    auto solve = [&](auto ic_) {
        constexpr int I = decltype(ic_)::value;
        // D_I = (I + N_II diag(beta)_I)^{-1} by forward substitution in fp32;
        // lane = (column col, row quad q)
        const int col = lane >> 2, q = lane & 3;
        // each column piece is read as two 8-byte loads: on gfx950 a 16-byte
        // LDS read costs several times two 8-byte reads
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        typedef __attribute__((address_space(3))) volatile const f32x2 vlds_f2;
        const auto lt = reinterpret_cast<__attribute__((address_space(3))) const float *>(
            (__attribute__((address_space(3))) const void *)&s.lt[I][4 * q]);
        auto ltcol = [&](int j) {
            const f32x2 lo = *reinterpret_cast<vlds_f2 *>(lt + j * LTS);
            const f32x2 hi = *reinterpret_cast<vlds_f2 *>(lt + j * LTS + 2);
            return f32x4{lo[0], lo[1], hi[0], hi[1]};
        };
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = (4 * q + r == col) ? 1.f : 0.f;
        // The columns of L do not depend on X: each is read PF steps before
        // its use, so the sweep does not wait on LDS latency.
        constexpr int PF = 3;
        f32x4 lw[PF + 1];
#pragma unroll
        for (int j = 0; j < PF; ++j) lw[j] = ltcol(j);
        auto sweep = [&](auto jc) {
            constexpr int j = decltype(jc)::value;
            if constexpr (j + PF < 15) lw[(j + PF) % (PF + 1)] = ltcol(j + PF);
            const f32x4 lj = lw[j % (PF + 1)];                           // L[4q + r][j]
            const float xj = quad_bcast<j / 4>(x[j % 4]);                // X[j][col]
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = fmaf(-lj[r], xj, x[r]);
        };
        static_for<15>(sweep);
        // D: element (row, col) goes to A-operand lane (col / 4) * 16 + row,
        // slot col % 4 (the scan scales its columns by -gamma for the state
        // term)
        __bf16 *dt = reinterpret_cast<__bf16 *>(&D.dtil[I][0]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = ((col >> 2) * 16 + 4 * q + r) * 4 + (col & 3);
            dt[e] = static_cast<__bf16>(x[r]);
        }
        // M_Ij = -D_I G~_Ij diag(beta)_j, computed transposed (A = -(G~
        // diag(beta))^T from the accumulators, B = D_I^T from its A-operand
        // fragment) so the result comes out in A-operand order
        if constexpr (I > 0) {
            if constexpr (I == 3) {  // blocks (3,0), (3,1), (3,2) from waves 0, 1
#pragma unroll
                for (int j = 0; j < 3; ++j) gneg[j] = s.gx[j][lane];
            }
            wave_lds_fence();  // this wave's D~_I pieces before the fragment read
            const bf16x4 dfrag = D.dtil[I][lane];
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < I; ++j) D.mij[lower_block(I, j)][lane] = bf4(mfma16(gneg[j], dfrag, zero));
        }
    };
    if (w == 0) solve(ic<0>{});
    else if (w == 1) solve(ic<1>{});
    else if (w == 2) solve(ic<2>{});
    else solve(ic<3>{});

    __syncthreads();

    // ---- the block, 16 bytes per thread and pass
    const uint4 *src = reinterpret_cast<const uint4 *>(&s.d);
    uint4 *dst = reinterpret_cast<uint4 *>(out + task);
    for (int i = tid; i < kDerPieces; i += NTD) dst[i] = src[i];
}

// ================================= scan =================================
template <int VARIANT, int DK, bool SIDE>
__global__ __launch_bounds__(NT8) void delta_chunked_wy_kernel(DeltaArgs a, const DerBlock *__restrict__ der,
                                                               unsigned int *status) {
    constexpr bool kDecay = VARIANT != kDeltaNet;
    constexpr int KS = DK + 8;
    constexpr int KSTEP = DK / 32;
    constexpr int KT = DK / 16;
    constexpr bool kGates2 = VARIANT == kGatedDeltaNet2;
    using Lds = WyLds<DK, kGates2>;
    __shared__ Lds s;

    const int T = static_cast<int>(a.T), H = static_cast<int>(a.H), dv = a.dv;
    const int slices = dv / BV;
    int head, slice;
    xcd_group_map(blockIdx.x, static_cast<int>(a.B * a.H), slices, head, slice);
    const int b = head / H, h = head % H;
    const int v0 = slice * BV;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lg = lane >> 4, lc = lane & 15;
    const int nchunks = (T + C - 1) / C;
    auto tok = [&](int t) { return (static_cast<int64_t>(b) * T + t) * H + h; };

    if (tid == 0) {
        s.ucount[0] = s.ucount[1] = 0u;
        s.scount[0] = s.scount[1] = 0u;
    }
    __syncthreads();  // counters visible before any role starts

    if (wave < 4) {
        // ========================= carry and output ==========================
        const bool is_carry = wave < 2;
        const int vt = wave & 1;
        f32x4 St[KT];
        const int vcol = v0 + 16 * vt + lc;
        const int64_t sbase = (static_cast<int64_t>(head) * dv + vcol) * DK;
        auto publish_state = [&]() {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) s.sh[vt][kt][lane] = bf4(St[kt]);
        };
        if (is_carry) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                if (a.state_in) {
                    const float4 x = *reinterpret_cast<const float4 *>(a.state_in + sbase + 16 * kt + 4 * lg);
                    St[kt] = f32x4{x.x, x.y, x.z, x.w};
                } else {
                    St[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
            publish_state();
        }
        // The output is computed transposed (Y^T = S Q^T + R^T Aqk^T, the same
        // fragments with the operands swapped), so lane (lg, lc) holds value
        // columns 4lg .. +3 of a tile for token lc of a row tile: one 8-byte
        // store per tile.
        const int64_t hdv = static_cast<int64_t>(H) * dv;
        auto step = [&](auto par, int c) {
            constexpr int P = decltype(par)::value;
            const typename Lds::Raw &R = s.raw[P];
            const DerBlock &D = s.der[P];
            bf16x8 bS[KSTEP];
            if (is_carry) {
                // Every read that does not depend on the state goes out first:
                // the key fragments of Z, then the value blocks and the solve
                // matrices, so their latency overlaps the Z products.
                bf16x8 kf[KSTEP][4];
#pragma unroll
                for (int p = 0; p < KSTEP; ++p)
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti) kf[p][ti] = row_frag2(kGates2 ? R.e : R.k, KS, 16 * ti, 32 * p, lane);
                bf16x4 vb[4], dt[4], dh[4], mj[NLB];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    vb[i] = col_gather4(R.v, Lds::VS, 16 * i, 16 * vt, lane);
                    dt[i] = D.dtil[i][lane];
                    // -D_i diag(gamma)_i: D_i's columns 16i + 4lg .. +3 times -gamma
                    if constexpr (kDecay) {
                        const float4 gm = *reinterpret_cast<const float4 *>(&D.gam[16 * i + 4 * lg]);
                        dh[i] = bf4(__builtin_convertvector(dt[i], f32x4) * f32x4{-gm.x, -gm.y, -gm.z, -gm.w});
                    } else {
                        dh[i] = -dt[i];
                    }
                }
#pragma unroll
                for (int i = 0; i < NLB; ++i) mj[i] = D.mij[i][lane];
#pragma unroll
                for (int p = 0; p < KSTEP; ++p) bS[p] = cat8(bf4(St[2 * p]), bf4(St[2 * p + 1]));
                // Z = E S^T, four row tiles
                f32x4 xp[4];
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) xp[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < KSTEP; ++p)
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti) xp[ti] = mfma32(kf[p][ti], bS[p], xp[ti]);
                // R_i = D_i V_i - D_i diag(gamma)_i Z_i + sum_{j<i} M_ij R_j
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                f32x4 u[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) u[i] = mfma16(dt[i], vb[i], zero);
#pragma unroll
                for (int i = 0; i < 4; ++i) u[i] = mfma16(dh[i], bf4(xp[i]), u[i]);
                bf16x4 ub[4];
                ub[0] = bf4(u[0]);
#pragma unroll
                for (int i = 1; i < 4; ++i) {
#pragma unroll
                    for (int j = 0; j < i; ++j) u[i] = mfma16(mj[lower_block(i, j)], ub[j], u[i]);
                    ub[i] = bf4(u[i]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) s.uh[vt][i][lane] = ub[i];
                lds_arrive(&s.ucount[vt], lane);
                state_update<KT>(St, R, D, ub, KS, lane);
                if (c + 1 < nchunks) {
                    lds_wait(&s.scount[vt], static_cast<unsigned int>(2 * (c + 1)), status);  // both output waves
                    publish_state();
                }
            } else {
                // Output wave vt takes token row tiles {0, 3} (vt = 0) or
                // {1, 2} (vt = 1) for both value tiles.  The lower blocks of
                // Aqk in its two rows are five either way, and they are the
                // only ones its rows need, so nothing passes between the
                // output waves; each reads half of the query fragments.
                bf16x8 bS0[KSTEP], bS1[KSTEP];
#pragma unroll
                for (int p = 0; p < KSTEP; ++p) {
                    bS0[p] = cat8(s.sh[0][2 * p][lane], s.sh[0][2 * p + 1][lane]);
                    bS1[p] = cat8(s.sh[1][2 * p][lane], s.sh[1][2 * p + 1][lane]);
                }
                lds_arrive(&s.scount[0], lane);  // the carries may overwrite sh from here on
                lds_arrive(&s.scount[1], lane);
                auto rows = [&](auto owc) {
                    constexpr int RT[2] = {decltype(owc)::value ? 1 : 0, decltype(owc)::value ? 2 : 3};
                    // Q S^T for both value tiles, and the blocks (i, j <= i) of
                    // K Q^T in rows i = RT[r]; block (i, j) comes out with lane
                    // (lg, lc) holding [s = 16j + 4lg + r][t = 16i + lc], the
                    // B-operand order of the product with R^T below
                    f32x4 xq[2][2], ka[2][4];
#pragma unroll
                    for (int r = 0; r < 2; ++r)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            ka[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                            if (j < 2) xq[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                        }
#pragma unroll
                    for (int p = 0; p < KSTEP; ++p) {
                        bf16x8 qf[2], kq[4];
#pragma unroll
                        for (int r = 0; r < 2; ++r) qf[r] = row_frag2(R.q, KS, 16 * RT[r], 32 * p, lane);
#pragma unroll
                        for (int j = 0; j <= RT[1]; ++j) kq[j] = row_frag2(R.k, KS, 16 * j, 32 * p, lane);
#pragma unroll
                        for (int r = 0; r < 2; ++r) {
                            xq[r][0] = mfma32(bS0[p], qf[r], xq[r][0]);
                            xq[r][1] = mfma32(bS1[p], qf[r], xq[r][1]);
                        }
#pragma unroll
                        for (int r = 0; r < 2; ++r)
#pragma unroll
                            for (int j = 0; j <= RT[r]; ++j) ka[r][j] = mfma32(kq[j], qf[r], ka[r][j]);
                    }
                    // Aqk = lower(Q K^T * Gamma) diag(beta): entry (t, s)
                    // scaled by 2^(g_t - g_s) beta_s = 2^(g_t - gb_s),
                    // exponent clamped at 0 so masked entries stay finite
                    // (below the diagonal it is at most log2 beta_s <= 0), and
                    // zero above the diagonal; and the first term of Y^T,
                    // S Q^T diag(gamma)
                    bf16x4 aq[2][4];
                    f32x4 y[2][2];
#pragma unroll
                    for (int r = 0; r < 2; ++r) {
                        const int i = RT[r];
                        const float gt = kDecay ? D.g[16 * i + lc] : 0.f;
#pragma unroll
                        for (int j = 0; j <= RT[r]; ++j) {
                            const float4 gs4 = *reinterpret_cast<const float4 *>(&D.gb[16 * j + 4 * lg]);
                            const float gs[4] = {gs4.x, gs4.y, gs4.z, gs4.w};
                            f32x4 x;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float v = kDecay ? ka[r][j][e] * exp2_fast(fminf(gt - gs[e], 0.f)) : ka[r][j][e] * gs[e];
                                x[e] = (j < i || 4 * lg + e <= lc) ? v : 0.f;
                            }
                            aq[r][j] = bf4(x);
                        }
                        const float gm = D.gam[16 * i + lc];
                        y[r][0] = xq[r][0] * gm;
                        y[r][1] = xq[r][1] * gm;
                    }
                    lds_wait(&s.ucount[0], static_cast<unsigned int>(c + 1), status);
                    lds_wait(&s.ucount[1], static_cast<unsigned int>(c + 1), status);
                    // Y^T += R^T Aqk^T, per value tile
                    const bf16x4 z4 = {};
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        bf16x4 ub[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) ub[i] = i <= RT[1] ? s.uh[t][i][lane] : z4;
                        const bf16x8 aU0 = cat8(ub[0], ub[1]), aU1 = cat8(ub[2], ub[3]);
#pragma unroll
                        for (int r = 0; r < 2; ++r) {
                            const int i = RT[r];
                            y[r][t] = mfma32(aU0, cat8(aq[r][0], i >= 1 ? aq[r][1] : z4), y[r][t]);
                            if (i >= 2) y[r][t] = mfma32(aU1, cat8(aq[r][2], i >= 3 ? aq[r][3] : z4), y[r][t]);
                        }
                    }
                    const int t0 = c * C;
                    uint16_t *yo = static_cast<uint16_t *>(a.out) + tok(t0) * dv +
                                   static_cast<uint32_t>(lc * hdv + v0 + 4 * lg);
#pragma unroll
                    for (int r = 0; r < 2; ++r)
#pragma unroll
                        for (int t = 0; t < 2; ++t)
                            if (t0 + 16 * RT[r] + lc < T)
                                *reinterpret_cast<bf16x4 *>(yo + static_cast<uint32_t>(16 * RT[r] * hdv + 16 * t)) =
                                    bf4(y[r][t]);
                    if constexpr (SIDE) {
                        // routing signal of this wave's token rows, off the
                        // carry's chain: the residuals R (bf16, as the carry
                        // published them) or the staged write targets (kept
                        // after the output's products, so its reads do not
                        // lengthen their register lifetimes)
                        __builtin_amdgcn_sched_barrier(0);
                        uint16_t *sb = static_cast<uint16_t *>(a.side) + tok(t0) * dv + v0;
                        const uint32_t h32 = static_cast<uint32_t>(hdv);
                        if (a.side_kind == kSideResidual) {
                            // R^T times an identity block on the matrix cores
                            // (exact: one product by 1, the rest by 0) lands R
                            // in y's layout, four columns of one token per
                            // lane: 8-byte row stores instead of scattered
                            // 2-byte ones.  Identity block for row tile i of
                            // its 32-token half, in the product's permuted
                            // reduction order (slots 4g .. 4g+3 hold tokens
                            // 4g + j of the half's first 16, slots 4 .. 7
                            // those of its second 16).
                            bf16x4 one4, zer4;
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                one4[j] = lc == 4 * lg + j ? static_cast<__bf16>(1.f) : static_cast<__bf16>(0.f);
                                zer4[j] = static_cast<__bf16>(0.f);
                            }
#pragma unroll
                            for (int t = 0; t < 2; ++t)
#pragma unroll
                                for (int r = 0; r < 2; ++r) {
                                    const int i = RT[r], hp = i >> 1;
                                    const bf16x8 aR = cat8(s.uh[t][2 * hp][lane], s.uh[t][2 * hp + 1][lane]);
                                    const f32x4 x = mfma32(aR, (i & 1) ? cat8(zer4, one4) : cat8(one4, zer4),
                                                           f32x4{0.f, 0.f, 0.f, 0.f});
                                    const int row = 16 * i + lc;
                                    if (t0 + row < T)
                                        *reinterpret_cast<bf16x4 *>(sb + static_cast<uint32_t>(row) * h32 + 16 * t + 4 * lg) =
                                            bf4(x);
                                }
                        } else {
#pragma unroll
                            for (int r = 0; r < 2; ++r)
#pragma unroll
                                for (int t = 0; t < 2; ++t) {
                                    const int row = 16 * RT[r] + lc;
                                    if (t0 + row < T)
                                        *reinterpret_cast<uint2 *>(sb + static_cast<uint32_t>(row) * h32 + 16 * t + 4 * lg) =
                                            *reinterpret_cast<const uint2 *>(&R.v[row * Lds::VS + 16 * t + 4 * lg]);
                                }
                        }
                    }
                };
                if (vt == 0) rows(ic<0>{});
                else rows(ic<1>{});
            }
            lds_barrier();
        };
        lds_barrier();  // chunk 0 staged, initial state published
        for (int c = 0; c < nchunks; c += 2) {
            step(ic<0>{}, c);
            if (c + 1 < nchunks) step(ic<1>{}, c + 1);
        }
        if (is_carry && a.state_out) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
                *reinterpret_cast<float4 *>(a.state_out + sbase + 16 * kt + 4 * lg) =
                    make_float4(St[kt][0], St[kt][1], St[kt][2], St[kt][3]);
        }
    } else {
        // ============================= producers =============================
        const int pw = wave - 4;  // stages token rows [16pw, 16pw + 16) of each chunk
        const uint16_t *gq = static_cast<const uint16_t *>(a.q);
        const uint16_t *gk = static_cast<const uint16_t *>(a.k);
        const uint16_t *gv = static_cast<const uint16_t *>(a.v);
        // Coalesced staging: a dk-wide bf16 row is DK/8 16-byte pieces, so
        // one load instruction covers 64*8/DK consecutive rows; a row of the
        // workgroup's 32 value columns is 4 pieces (16 rows per instruction).
        constexpr int PPR = DK / 8;             // 16-byte pieces per q/k row
        constexpr int RPI = 64 / PPR;           // rows per load instruction
        constexpr int NQK = 16 / RPI;           // instructions per producer per stream
        const uint32_t hdk = static_cast<uint32_t>(H * DK), hdv = static_cast<uint32_t>(H * dv);
        const int qrow = 16 * pw + lane / PPR;  // chunk row of this lane's first q/k piece
        const int vrow = 16 * pw + (lane >> 2);
        // Pieces of the derived block: 64pw + lane + 256j, j < 4, where they exist.
        const int dp0 = 64 * pw + lane;
        constexpr int NDP = (kDerPieces + 255) / 256;
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 *gder = reinterpret_cast<const u32x4 *>(der + static_cast<int64_t>(head) * nchunks);
        // Two staging sets: loads run two chunks ahead (Gated DeltaNet-2
        // stages two more streams, the erase and write gates, in each set).
        constexpr int NS = 2;
        constexpr int NQKG = kGates2 ? NQK : 1;
        const uint16_t *geb = static_cast<const uint16_t *>(a.erase_b);
        const uint16_t *gww = static_cast<const uint16_t *>(a.write_w);
        struct Stage {
            uint4 q[NQK], k[NQK], v;
            uint4 b[NQKG], w;  // erase / write gates (Gated DeltaNet-2)
            u32x4 d[NDP];      // pieces of the derived block
            uint32_t okm;      // bit i: row of q/k load i inside the sequence; bit NQK: v row
        };
        Stage st[NS];
        // Loads read clamped, always valid rows; rows past the end are replaced
        // by padding at commit, so no loaded value is consumed here and the
        // loads stay in flight until that chunk's staging.
        auto fetch = [&](auto par, int c) {
            Stage &g = st[decltype(par)::value % NS];
            const int t0 = c * C, last = T - 1 - t0;
            const int64_t base = tok(t0);
            const uint16_t *q0 = gq + base * DK, *k0 = gk + base * DK;
            g.okm = 0u;
#pragma unroll
            for (int i = 0; i < NQK; ++i) {
                const int r = qrow + RPI * i;
                g.okm |= (r <= last ? 1u : 0u) << i;
                const uint32_t o = static_cast<uint32_t>(min(r, last)) * hdk + (lane % PPR) * 8;
                g.q[i] = *reinterpret_cast<const uint4 *>(q0 + o);
                g.k[i] = *reinterpret_cast<const uint4 *>(k0 + o);
                if constexpr (kGates2) g.b[i] = *reinterpret_cast<const uint4 *>(geb + base * DK + o);
            }
            g.okm |= (vrow <= last ? 1u : 0u) << NQK;
            // Row product and column offset stay separate instructions: fused,
            // they become a 64-bit multiply-add whose undefined upper addend
            // half may be allocated to an in-flight load's destination, and
            // the load-counter wait for that register would drain the other
            // staging set.
            uint32_t ov = static_cast<uint32_t>(min(vrow, last)) * hdv;
            asm("" : "+v"(ov));
            ov += v0 + 8 * (lane & 3);
            g.v = *reinterpret_cast<const uint4 *>(gv + base * dv + ov);
            if constexpr (kGates2) g.w = *reinterpret_cast<const uint4 *>(gww + base * dv + ov);
            const u32x4 *src = gder + static_cast<int64_t>(c) * kDerPieces;
#pragma unroll
            for (int j = 0; j < NDP; ++j) g.d[j] = src[min(dp0 + 256 * j, kDerPieces - 1)];
        };
        auto commit = [&](auto par) {
            typename Lds::Raw &R = s.raw[decltype(par)::value];
            const Stage &g = st[decltype(par)::value % NS];
#pragma unroll
            for (int i = 0; i < NQK; ++i) {
                const int row = qrow + RPI * i;
                const uint32_t m = 0u - ((g.okm >> i) & 1u);
                *reinterpret_cast<uint4 *>(&R.q[row * KS + (lane % PPR) * 8]) = masked(g.q[i], m);
                *reinterpret_cast<uint4 *>(&R.k[row * KS + (lane % PPR) * 8]) = masked(g.k[i], m);
                if constexpr (kGates2)
                    *reinterpret_cast<uint4 *>(&R.e[row * KS + (lane % PPR) * 8]) = masked(mul8(g.k[i], g.b[i]), m);
            }
            const uint32_t mv = 0u - ((g.okm >> NQK) & 1u);
            *reinterpret_cast<uint4 *>(&R.v[vrow * Lds::VS + 8 * (lane & 3)]) =
                masked(kGates2 ? mul8(g.v, g.w) : g.v, mv);
            u32x4 *dd = reinterpret_cast<u32x4 *>(&s.der[decltype(par)::value]);
#pragma unroll
            for (int j = 0; j < NDP; ++j)
                if (dp0 + 256 * j < kDerPieces) dd[dp0 + 256 * j] = g.d[j];
        };
        // Preparing chunk n: stage it from its set, then refill that set with
        // chunk n + NS.  The refill is issued on every path (past the end it
        // reloads the last chunk, which is never staged), so the loads in
        // flight always form the same queue and the staging waits only for
        // the older set.
        auto prepare = [&](auto par, int n) {
            commit(par);
            fetch(par, min(n + NS, nchunks - 1));
        };
        if (nchunks > 0) {
            fetch(ic<0>{}, 0);
            if constexpr (NS == 2) fetch(ic<1>{}, min(1, nchunks - 1));
            prepare(ic<0>{}, 0);
        }
        lds_barrier();  // chunk 0 staged
        // One barrier per chunk, as in the carry and output loop.  The loop
        // has a single exit and every trip runs both prepares, so each path
        // around it issues the same loads in the same order and a staging
        // set's wait leaves the other set in flight.
        int c = 0;
        for (; c + 2 < nchunks; c += 2) {
            prepare(ic<1>{}, c + 1);  // during chunk c: chunk c + 1 (buffers 1)
            lds_barrier();
            prepare(ic<0>{}, c + 2);  // during chunk c + 1: chunk c + 2 (buffers 0)
            lds_barrier();
        }
        if (c + 1 < nchunks) {  // chunks c and c + 1 remain
            prepare(ic<1>{}, c + 1);
            lds_barrier();
            lds_barrier();
        } else if (c < nchunks) {  // chunk c remains
            lds_barrier();
        }
    }
}

template <int VARIANT, int DK>
hipError_t launch_dk(const DeltaArgs &a, hipStream_t stream) {
    const int64_t nchunks = (a.T + C - 1) / C;
    const int64_t tasks = a.B * a.H * nchunks;
    const unsigned blocks = static_cast<unsigned>(a.B * a.H * (a.dv / BV));
    unsigned int *status = static_cast<unsigned int *>(a.ws);
    DerBlock *der = reinterpret_cast<DerBlock *>(static_cast<char *>(a.ws) + kStatusBytes);
    if (tasks > 0)
        delta_chunked_derive_kernel<VARIANT, DK><<<static_cast<unsigned>(tasks), NTD, 0, stream>>>(a, der, status);
    if (a.side)
        delta_chunked_wy_kernel<VARIANT, DK, true><<<blocks, NT8, 0, stream>>>(a, der, status);
    else
        delta_chunked_wy_kernel<VARIANT, DK, false><<<blocks, NT8, 0, stream>>>(a, der, status);
    return hipGetLastError();
}

template <int VARIANT>
hipError_t launch_var(const DeltaArgs &a, hipStream_t stream) {
    switch (a.dk) {
        case 64: return launch_dk<VARIANT, 64>(a, stream);
        case 128: return launch_dk<VARIANT, 128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

namespace {
// the bf16 schedule of this file; every other DeltaNet / Gated DeltaNet /
// Gated DeltaNet-2 shape takes the fp32 chunked form (delta_chunked_f32.hip)
bool bf16_schedule(const DeltaArgs &a) {
    return a.dtype == kBF16 && (a.dk == 64 || a.dk == 128) && a.dv % BV == 0;
}
}  // namespace

bool delta_chunked_supported(const DeltaArgs &a) {
    if (a.variant == kKimiDelta) return kda_chunked_supported(a);
    return bf16_schedule(a) || delta_f32_chunked_supported(a);
}

bool delta_chunked_workspace(const DeltaArgs &a, size_t *bytes) {
    if (a.variant == kKimiDelta) return kda_chunked_workspace(a, bytes);
    if (!bf16_schedule(a)) return delta_f32_chunked_workspace(a, bytes);
    const int64_t tasks = a.B * a.H * ((a.T + C - 1) / C);
    if (tasks > 0x7fffffff) return false;
    *bytes = kStatusBytes + static_cast<size_t>(tasks) * sizeof(DerBlock);
    return true;
}

hipError_t launch_delta_chunked(const DeltaArgs &a, hipStream_t stream) {
    if (!delta_chunked_supported(a)) return hipErrorNotSupported;
    if (a.variant != kKimiDelta && !bf16_schedule(a)) return launch_delta_f32_chunked(a, stream);
    switch (a.variant) {
        case kDeltaNet: return launch_var<kDeltaNet>(a, stream);
        case kGatedDeltaNet: return launch_var<kGatedDeltaNet>(a, stream);
        case kGatedDeltaNet2: return launch_var<kGatedDeltaNet2>(a, stream);
        case kKimiDelta: return launch_kda_chunked(a, stream);
    }
    return hipErrorNotSupported;
}

}  // namespace lam
