// vla_chunked.hip -- chunked VLA scan on gfx950 fp32 matrix cores.
//
// The rules ("Technical summary: Variational Linear Attention (VLA)",
// sections 2.2-2.3): per token the inverse penalty takes a rank-1
// Sherman-Morrison downdate A <- A - z z^T / (1 + p.z) with z = A p, the gate
// is the unit vector along A khat, and the state writes its residual along
// the gate, S <- S + (v - S khat) alphahat^T; keys and queries pass through
// ELU+1 and unit normalisation; y = S qhat.
//
// A is the inverse of the penalty M = A_0^{-1} + sum_s p_s p_s^T (section
// 2.2: the Sherman-Morrison step keeps A = M^{-1} exactly), so the penalty at
// any token is a prefix sum, and A there is its inverse.  That makes the
// gates parallel over the sequence: it is cut into segments, the inverse
// penalty at each segment start is formed directly, and the rank-1 steps
// then run inside the segments concurrently.  The gates do not depend on
// the state, so the state scan runs afterwards, split over value rows.
//
// Four kernels per call (segments of SEG tokens, chunks of C = 16 tokens):
//   gram:    per (b, h, segment): G = P^T P over the segment's tokens (fp32).
//   inverse: per (b, h, segment > 0): M = A_0^{-1} + sum of the earlier
//            segments' G, inverted by Gauss-Jordan in fp64 (M is symmetric
//            positive definite, so no pivoting) -> A at the segment start.
//   alpha:   per (b, h, segment): from that A, the chunked rank-1 steps over
//            the segment's chunks (rows = tokens; A at the chunk start):
//              Pa = P A^T, KA = Khat A^T, F = Z X^T with X = [P; Khat]:
//              F_t = (Pa X^T)_t - sum_{s<t} c_ts F_s, c_ts = F_s[p_t] / D_s,
//              D_t = 1 + F_t[p_t]          (z_t = A_{t-1} p_t, D_t = 1 + p_t.z_t)
//              Z = (I + C)^{-1} Pa, N = KA - E Z with E_ts = F_s[khat_t] / D_s
//              (s <= t), alphahat_t = N_t / |N_t|, A <- A - Z^T D^{-1} Z;
//            then the state-independent operands of each chunk's state step,
//            with Tc = (I + strict(Khat Ahat^T))^{-1} and Aq = lower(Qhat Ahat^T):
//              Ktil = Tc Khat, Qtil = Qhat - Aq Ktil, Tc and Aq Tc,
//            written with alphahat to a per-chunk record.
//   state:   per (b, h, 16 value rows of S): the generalised delta scan
//              U = Tc (V - Khat S^T) = Tc V - Ktil S^T,
//              Y = Qhat S^T + Aq U = Qtil S^T + (Aq Tc) V,  S <- S + U^T Ahat,
//            with the key dimension of S^T split over the workgroup's D/16
//            waves (one 16 x 16 accumulator tile each) and the partial
//            products summed through LDS, one barrier per chunk.  Tc V and
//            (Aq Tc) V do not depend on the state, so the only products on
//            the chunk-to-chunk chain are Ktil S^T, Qtil S^T and the update.
// The last segment's alpha workgroup writes A_out; the state workgroups
// write S_out.  The state kernel and the chunk record are in chunk_f32.h,
// shared with the fp32 form of the delta-rule family.
#include "chunk_f32.h"

namespace lam {
namespace {

__device__ __forceinline__ float elu1(float x) { return x > 0.f ? x + 1.f : __expf(x); }

constexpr int NT64 = 64;  // lanes per wave

// Tokens per segment of the inverse-penalty chain.  Each segment past the
// first costs one d x d inversion; longer segments lengthen the chain inside
// each alpha workgroup.
__host__ __device__ constexpr int seg_len(int D) { return D <= 32 ? 128 : 256; }

// Workspace layout of one call (after the status block): G and the segment-
// start inverses, one D x D fp32 matrix per (b, h, segment), then the chunk
// records per (b, h, chunk).
struct VlaLayout {
    int64_t nseg, nch;
    size_t g_off, a_off, rec_off, bytes;
};
template <int D>
VlaLayout vla_layout(int64_t B, int64_t T, int64_t H) {
    VlaLayout L;
    L.nseg = (T + seg_len(D) - 1) / seg_len(D);
    L.nch = (T + VC - 1) / VC;
    const size_t mat = static_cast<size_t>(B * H * L.nseg) * D * D * sizeof(float);
    auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    L.g_off = kStatusBytes;
    L.a_off = up(L.g_off + mat);
    L.rec_off = up(L.a_off + mat);
    L.bytes = L.rec_off + static_cast<size_t>(B * H * L.nch) * sizeof(ChunkRec<D>);
    return L;
}

// ================================ gram ================================
// One workgroup of D/16 waves per (b, h, segment s < nseg - 1); wave w forms
// column tile w of G = P^T P over the segment, on and below the diagonal
// blocks (G is symmetric: the blocks above are written as their mirrors).  Chunk tiles go through LDS
// transposed (PT[channel][token]), so both operands are float4 reads.
template <typename IO, int D>
__global__ __launch_bounds__(64 * (D / 16)) void vla_gram_kernel(VlaArgs a, float *__restrict__ G, int nseg,
                                                                  unsigned int *status) {
    constexpr int NW = D / 16, NT = 64 * NW, NQ = D / 16, TS = VC + 4, EPT = VC * D / NT;
    constexpr int SEG = seg_len(D);
    __shared__ float pt[D * TS];
    const int T = static_cast<int>(a.T), H = static_cast<int>(a.H);
    const int nm1 = nseg - 1;
    const int head = blockIdx.x / nm1, sg = blockIdx.x % nm1;
    const int b = head / H, h = head % H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, i = lane & 15;
    if (blockIdx.x == 0 && tid == 0) *status = 0u;  // first kernel of the call
    const int t0 = sg * SEG, t1 = min(T, t0 + SEG);
    auto tok = [&](int t) { return ((static_cast<int64_t>(b) * T + t) * H + h) * D; };
    float rp[EPT];
    auto fetch = [&](int c0) {
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const int e = tid + NT * u, t = e / D, j = e % D;
            rp[u] = c0 + t < t1 ? IO::ld(a.p, tok(c0 + t) + j) : 0.f;
        }
    };
    f32x4 acc[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    fetch(t0);
    for (int c0 = t0; c0 < t1; c0 += VC) {
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const int e = tid + NT * u;
            pt[(e % D) * TS + e / D] = rp[u];
        }
        lds_sync();
        if (c0 + VC < t1) fetch(c0 + VC);
        const f32x4 bw = lds4(&pt[(16 * w + i) * TS + 4 * g]);  // P[4g + m][16w + i]
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            if (q < w) continue;  // G is symmetric: blocks on and below the diagonal
            const f32x4 aq4 = lds4(&pt[(16 * q + i) * TS + 4 * g]);  // P[4g + m][16q + i]
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[q] = mfma4(aq4[m], bw[m], acc[q]);
        }
        lds_sync();
    }
    // acc[q] lane (g, i): G[16q + 4g + r][16w + i] for blocks q >= w; the
    // blocks above the diagonal are their mirror images (four consecutive
    // floats of row 16w + i per lane)
    float *out = G + (static_cast<int64_t>(head) * nseg + sg) * D * D;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
        if (q >= w) {
#pragma unroll
            for (int r = 0; r < 4; ++r) out[(16 * q + 4 * g + r) * D + 16 * w + i] = acc[q][r];
            if (q > w)
                *reinterpret_cast<float4 *>(&out[(16 * w + i) * D + 16 * q + 4 * g]) =
                    make_float4(acc[q][0], acc[q][1], acc[q][2], acc[q][3]);
        }
}

// =============================== inverse ===============================
// In-place Gauss-Jordan inversion of the symmetric positive definite D x D
// matrix held in registers by a 16 x 16 grid of threads (thread (ti, tj) owns
// rows ti + 16a, columns tj + 16c).  Step k: the owners of row k and column k
// publish them; every element then takes
//   M[k][k] = 1/p, M[k][j] = M[k][j]/p, M[i][k] = -M[i][k]/p,
//   M[i][j] -= M[i][k] M[k][j] / p   (p = M[k][k], old values throughout),
// written as one rank-1 update (below).  M's eigenvalues lie in [1, 1 + the
// largest of sum p p^T] (A_0 has eigenvalues in (0, 1]), so the pivots stay
// well away from zero.
// The row and column buffers alternate by step parity (16 steps per block,
// so the parity also alternates across blocks), so one barrier per step
// orders both their writes and the reads of the step before.
template <int D>
__device__ __forceinline__ void gj_invert(double (&M)[D / 16][D / 16], double (*rowbuf)[D], double (*colbuf)[D],
                                          int ti, int tj) {
    constexpr int RD = D / 16;
    // pivot k = 16 kq + kr: the block index kq is a compile-time constant in
    // each unrolled copy, so M is only ever indexed statically (a runtime
    // index would move it to scratch memory)
    auto steps = [&](auto kqc) {
        constexpr int kq = decltype(kqc)::value;
#pragma unroll 1
        for (int kr = 0; kr < 16; ++kr) {
            const int k = 16 * kq + kr, pb = kr & 1;
            if (ti == kr) {
#pragma unroll
                for (int c = 0; c < RD; ++c) rowbuf[pb][tj + 16 * c] = M[kq][c];
            }
            if (tj == kr) {
#pragma unroll
                for (int r = 0; r < RD; ++r) colbuf[pb][ti + 16 * r] = M[r][kq];
            }
            lds_sync();
            // 1/p by the hardware reciprocal and two Newton steps (each
            // squares the relative error: 2^-23 -> 2^-46 -> below fp64 rounding)
            const double pv = rowbuf[pb][k];
            double ip = __builtin_amdgcn_rcp(pv);
            ip = fma(ip, fma(-pv, ip, 1.0), ip);
            ip = fma(ip, fma(-pv, ip, 1.0), ip);
            // The whole step is one rank-1 update M -= c r^T, with
            //   c_i = M[i][k] (i != k), c_k = p - 1,
            //   r_j = M[k][j] / p (j != k), r_k = 1 + 1/p,
            // which gives row k -> M[k][j] / p, column k -> -M[i][k] / p and
            // M[k][k] -> p - (p - 1)(1 + 1/p) = 1/p.
            double rk[RD], ck[RD];
#pragma unroll
            for (int c = 0; c < RD; ++c) {
                const bool isk = c == kq && tj == kr;
                rk[c] = isk ? 1.0 + ip : rowbuf[pb][tj + 16 * c] * ip;
            }
#pragma unroll
            for (int r = 0; r < RD; ++r) {
                const bool isk = r == kq && ti == kr;
                ck[r] = isk ? pv - 1.0 : colbuf[pb][ti + 16 * r];
            }
#pragma unroll
            for (int r = 0; r < RD; ++r)
#pragma unroll
                for (int c = 0; c < RD; ++c) M[r][c] = fma(-ck[r], rk[c], M[r][c]);
        }
    };
    static_for<RD>(steps);
}

// One workgroup of 256 threads per (b, h, segment s >= 1): M = A_0^{-1} +
// sum_{s' < s} G_s' in fp64, then A_s = M^{-1} (written as fp32).
template <int D>
__global__ __launch_bounds__(256) void vla_inverse_kernel(VlaArgs a, const float *__restrict__ G,
                                                          float *__restrict__ Aseg, int nseg) {
    constexpr int RD = D / 16;
    __shared__ double rowbuf[2][D], colbuf[2][D];
    const int nm1 = nseg - 1;
    int head, sm1;
    xcd_group_map(blockIdx.x, static_cast<int>(a.B * a.H), nm1, head, sm1);
    const int sg = sm1 + 1;
    const int tid = threadIdx.x, ti = tid >> 4, tj = tid & 15;
    const int64_t sb = static_cast<int64_t>(head) * D * D;
    double M[RD][RD];
    if (a.A_in) {  // A_0^{-1}
#pragma unroll
        for (int r = 0; r < RD; ++r)
#pragma unroll
            for (int c = 0; c < RD; ++c) M[r][c] = a.A_in[sb + (ti + 16 * r) * D + tj + 16 * c];
        gj_invert<D>(M, rowbuf, colbuf, ti, tj);
    } else {
#pragma unroll
        for (int r = 0; r < RD; ++r)
#pragma unroll
            for (int c = 0; c < RD; ++c) M[r][c] = (ti + 16 * r == tj + 16 * c) ? 1.0 : 0.0;
    }
    // the earlier segments' G
    const float *g0 = G + static_cast<int64_t>(head) * nseg * D * D;
#pragma unroll 1
    for (int s = 0; s < sg; ++s) {
        const float *gs = g0 + static_cast<int64_t>(s) * D * D;
#pragma unroll
        for (int r = 0; r < RD; ++r)
#pragma unroll
            for (int c = 0; c < RD; ++c) M[r][c] += gs[(ti + 16 * r) * D + tj + 16 * c];
    }
    gj_invert<D>(M, rowbuf, colbuf, ti, tj);
    float *out = Aseg + (static_cast<int64_t>(head) * nseg + sg) * D * D;
#pragma unroll
    for (int r = 0; r < RD; ++r)
#pragma unroll
        for (int c = 0; c < RD; ++c) out[(ti + 16 * r) * D + tj + 16 * c] = static_cast<float>(M[r][c]);
}

// ================================ alpha ================================
template <int D>
struct AlphaLds {
    static constexpr int DS = D + 4;  // row stride of the token-row tiles
    static constexpr int TS = VC + 4; // row stride of the transposed tiles
    // token-row tiles, double-buffered: chunk c is consumed while chunk c + 1
    // is staged and its features are computed
    alignas(16) float p[2][VC * DS], kh[2][VC * DS], qh[2][VC * DS];
    alignas(16) float pa[VC * DS];      // P A^T
    alignas(16) float ah[VC * DS];      // alphahat rows
    alignas(16) float zt[D * TS];       // Z^T
    alignas(16) float g0t[2 * VC * TS]; // (Pa X^T)^T: column c of Pa X^T as a row
    alignas(16) float e[VC * TS];       // E, rows t
    alignas(16) float lt[VC * VLTS];    // strictly lower matrix by column (C, then strict(Khat Ahat^T))
    alignas(16) f32x4 wop[64];          // (I + C)^{-1}, A-operand order
    alignas(16) f32x4 top[64];          // (I + strict(Khat Ahat^T))^{-1}, A-operand order
    alignas(16) f32x4 aq[64];           // lower(Qhat Ahat^T), A-operand order
    alignas(16) float rd[VC];           // 1 / D_t
    alignas(16) float part[D / 16][VC]; // per-wave partial |N_t|^2
};

// Tiles of A^T per wave in the alpha kernel.  At D = 96 the six column tiles
// go two to a wave over three waves, and a fourth wave runs the serial parts
// (the Sherman-Morrison recurrence and Tc): four waves spread evenly over the
// SIMDs, so two workgroups fit on a compute unit (six one-tile waves put two
// waves on each of SIMDs 0 and 1, and two such workgroups do not fit).
template <int D>
__host__ __device__ constexpr int alpha_tpw() { return D == 96 ? 2 : 1; }
template <int D>
__host__ __device__ constexpr int alpha_waves() { return D / 16 / alpha_tpw<D>() + (alpha_tpw<D>() > 1 ? 1 : 0); }

// One workgroup per (b, h, segment).  Tile wave w keeps column tiles
// w TPW .. w TPW + TPW - 1 of A^T as fp32 accumulator tiles.
template <typename IO, int D>
__device__ __forceinline__ void vla_alpha_body(AlphaLds<D> &s, const VlaArgs &a, const float *__restrict__ Aseg,
                                               ChunkRec<D> *__restrict__ rec, int nseg, unsigned int *status) {
    constexpr int NW = D / 16, NQ = D / 16;
    constexpr int TPW = alpha_tpw<D>(), NTW = NW / TPW, NWV = alpha_waves<D>(), NT = 64 * NWV;
    constexpr int FW = TPW > 1 ? NTW : 0;  // the wave that runs the recurrence for F and forms Tc
    constexpr int DS = AlphaLds<D>::DS, TS = AlphaLds<D>::TS;
    constexpr int SEG = seg_len(D);

    const int T = static_cast<int>(a.T), H = static_cast<int>(a.H);
    const int head = blockIdx.x / nseg, sg = blockIdx.x % nseg;
    const int b = head / H, h = head % H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, i = lane & 15;
    const int64_t sb = static_cast<int64_t>(head) * D * D;
    const bool tiles = w < NTW;
    // this lane's column of tile tw of the wave (clamped for the helper wave, which has none)
    auto colof = [&](int tw) { return 16 * (min(w, NTW - 1) * TPW + tw) + i; };
    const int seg0 = sg * SEG, seg1 = min(T, seg0 + SEG);
    const int nch = (T + VC - 1) / VC;
    if (nseg == 1 && blockIdx.x == 0 && tid == 0) *status = 0u;  // first kernel of the call

    // A^T column tiles: AT[tw][q] = A^T[16q + 4g + r][col] = A[col][16q + 4g + r]
    const float *a0 = sg > 0 ? Aseg + (static_cast<int64_t>(head) * nseg + sg) * D * D
                             : (a.A_in ? a.A_in + sb : nullptr);
    f32x4 AT[TPW][NQ];
#pragma unroll
    for (int tw = 0; tw < TPW; ++tw) {
        const int col = colof(tw);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            if (a0) {
                const float4 x = *reinterpret_cast<const float4 *>(a0 + static_cast<int64_t>(col) * D + 16 * q + 4 * g);
                AT[tw][q] = f32x4{x.x, x.y, x.z, x.w};
            } else {
                f32x4 x;
#pragma unroll
                for (int r = 0; r < 4; ++r) x[r] = (16 * q + 4 * g + r == col) ? 1.f : 0.f;
                AT[tw][q] = x;
            }
        }
    }

    // raw inputs of one chunk staged in registers: element e = tid + NT * u of
    // each 16 x D tile (token e / D, channel e % D)
    constexpr int EPT = VC * D / NT;
    static_assert(EPT * NT == VC * D, "staging covers the tile exactly");
    float rq[EPT], rk[EPT], rp[EPT];
    auto tok = [&](int t) { return ((static_cast<int64_t>(b) * T + t) * H + h) * D; };
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
            const uint32_t o = t < n ? eoff[u] : static_cast<uint32_t>((n - 1) * H * D + e % D);
            rq[u] = IO::ld(a.q, base + o);
            rk[u] = IO::ld(a.k, base + o);
            rp[u] = IO::ld(a.p, base + o);
        }
    };
    // staged registers into buffer bi (rows past n: p = 0, features zeroed)
    auto stage = [&](int bi, int n) {
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const int e = tid + NT * u, t = e / D, j = e % D;
            s.p[bi][t * DS + j] = t < n ? rp[u] : 0.f;
            s.kh[bi][t * DS + j] = rk[u];
            s.qh[bi][t * DS + j] = rq[u];
        }
    };
    // khat (or qhat) = unit(ELU(x) + 1) in place for the 16 rows of tile X,
    // zero past row n, by one wave: lane (g, i) maps token i, channels
    // 16q + 4g .. 16q + 4g + 3; the squared norm adds the lane's terms, then
    // the four lane groups' partial sums (the same bits in every lane).
    auto features = [&](float *X, int n) {
        f32x4 f[NQ];
        float ss = 0.f;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            f32x4 x = lds4(&X[i * DS + 16 * q + 4 * g]);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                x[m] = elu1(x[m]);
                ss = fmaf(x[m], x[m], ss);
            }
            f[q] = x;
        }
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        const float inv = __builtin_amdgcn_rsqf(ss);
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            *reinterpret_cast<f32x4 *>(&X[i * DS + 16 * q + 4 * g]) =
                i < n ? f[q] * inv : f32x4{0.f, 0.f, 0.f, 0.f};
    };
    // waves mapping the next chunk's keys and queries during the recurrence
    constexpr int WKF = FW == 1 ? 2 : 1;
    constexpr int WQF = NWV > 2 ? (FW == 2 ? 3 : 2) : 1;
    if (seg0 < seg1) {
        fetch(seg0);
        stage(0, min(VC, seg1 - seg0));
        fetch(seg0 + VC);
        lds_sync();
        if (w == 0) features(s.kh[0], min(VC, seg1 - seg0));
        if (w == 1) features(s.qh[0], min(VC, seg1 - seg0));
    }

    for (int c0 = seg0; c0 < seg1; c0 += VC) {
        const int n = min(VC, seg1 - c0), n1 = max(0, min(VC, seg1 - c0 - VC));  // rows of this chunk, of the next
        const int cb = ((c0 - seg0) / VC) & 1, nb = cb ^ 1;
        const float *P = s.p[cb], *KH = s.kh[cb], *QH = s.qh[cb];
        ChunkRec<D> &R = rec[static_cast<int64_t>(head) * nch + c0 / VC];
        // ---- stage chunk c + 1 into the other buffer, refill the registers
        stage(nb, n1);
        fetch(c0 + 2 * VC);
        lds_sync();
        // ---- products against the chunk-start inverse penalty (per tile):
        // Pa = P A^T, KA = Khat A^T (two accumulators each: even and odd
        // reduction steps, so the dependent chains are half as long)
        const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
        f32x4 pa[TPW], ka[TPW];
        if (tiles) {
            f32x4 pa2[TPW][2], ka2[TPW][2];
#pragma unroll
            for (int tw = 0; tw < TPW; ++tw) pa2[tw][0] = pa2[tw][1] = ka2[tw][0] = ka2[tw][1] = zero4;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const f32x4 pr = lds4(&P[i * DS + 16 * q + 4 * g]);
                const f32x4 kr = lds4(&KH[i * DS + 16 * q + 4 * g]);
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int tw = 0; tw < TPW; ++tw) {
                        pa2[tw][m & 1] = mfma4(pr[m], AT[tw][q][m], pa2[tw][m & 1]);
                        ka2[tw][m & 1] = mfma4(kr[m], AT[tw][q][m], ka2[tw][m & 1]);
                    }
            }
#pragma unroll
            for (int tw = 0; tw < TPW; ++tw) {
                pa[tw] = pa2[tw][0] + pa2[tw][1];
                ka[tw] = ka2[tw][0] + ka2[tw][1];
                const int col = colof(tw);
#pragma unroll
                for (int r = 0; r < 4; ++r) s.pa[(4 * g + r) * DS + col] = pa[tw][r];
            }
        }
        lds_sync();
        // ---- Pa X^T (16 x 32), waves 0 and 1: column c of it stored as row c of g0t
        if (w < 2) {
            const float *xs = w == 0 ? P : KH;
            f32x4 g2[2] = {zero4, zero4};
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const f32x4 ar = lds4(&s.pa[i * DS + 16 * q + 4 * g]);
                const f32x4 br = lds4(&xs[i * DS + 16 * q + 4 * g]);
#pragma unroll
                for (int m = 0; m < 4; ++m) g2[m & 1] = mfma4(ar[m], br[m], g2[m & 1]);
            }
            const f32x4 g0 = g2[0] + g2[1];
            // g0 lane (g, i): (Pa X^T)[t = 4g + r][16w + i]
            *reinterpret_cast<f32x4 *>(&s.g0t[(16 * w + i) * TS + 4 * g]) = g0;
        }
        lds_sync();
        // ---- wave FW: the recurrence for F, then Z's coefficients inverted
        if (w == FW) {
            // lane c < 32 keeps column c of F: F[s] = F_s[c].  Right-looking:
            // once F_s is final, its term -c_ts F_s (c_ts = F_s[p_t] / D_s,
            // column t of F_s, held by lane t) goes into every later row at
            // once, so each step's critical path is one row's last update.
            const int c = lane & 31;
            float acc[VC], F[VC], rdv[VC];
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) {
                const f32x4 x = lds4(&s.g0t[c * TS + 4 * t4]);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[4 * t4 + r] = x[r];
            }
#pragma unroll
            for (int s2 = 0; s2 < VC; ++s2) {
                F[s2] = acc[s2];
                const float ds = 1.f + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(F[s2]), s2));
                rdv[s2] = __builtin_amdgcn_rcpf(ds);
#pragma unroll
                for (int t = s2 + 1; t < VC; ++t) {
                    const float cts = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(F[s2]), t)) * rdv[s2];
                    acc[t] = fmaf(-cts, F[s2], acc[t]);
                }
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
            // meanwhile other waves map the features of chunk c + 1
            if (w == WKF) features(s.kh[nb], n1);
            if (w == WQF) features(s.qh[nb], n1);
        }
        lds_sync();
        // ---- Z = (I + C)^{-1} Pa, N = KA - E Z (per tile); Z^T to LDS; |N_t|^2 partials
        f32x4 z[TPW], nn[TPW];
        if (tiles) {
            const f32x4 wa = s.wop[lane];
            const f32x4 ea = lds4(&s.e[i * TS + 4 * g]);
#pragma unroll
            for (int tw = 0; tw < TPW; ++tw) {
                z[tw] = zero4;
                nn[tw] = ka[tw];
#pragma unroll
                for (int m = 0; m < 4; ++m) z[tw] = mfma4(wa[m], pa[tw][m], z[tw]);
#pragma unroll
                for (int m = 0; m < 4; ++m) nn[tw] = mfma4(-ea[m], z[tw][m], nn[tw]);
                const int col = colof(tw);
                *reinterpret_cast<f32x4 *>(&s.zt[col * TS + 4 * g]) = z[tw];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float sq = group_sum<16>(nn[tw][r] * nn[tw][r]);
                    if (i == 0) s.part[w * TPW + tw][4 * g + r] = sq;
                }
            }
        }
        lds_sync();
        // ---- alphahat (per tile) to LDS by rows and to the record; A^T -= Z^T D^{-1} Z
        if (tiles) {
            float rn[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * g + r;
                float ss = 0.f;
#pragma unroll
                for (int u = 0; u < NW; ++u) ss += s.part[u][t];
                rn[r] = t < n ? __builtin_amdgcn_rsqf(ss) : 0.f;
            }
            const f32x4 rd4 = lds4(&s.rd[4 * g]);
#pragma unroll
            for (int tw = 0; tw < TPW; ++tw) {
                const int col = colof(tw);
                f32x4 ah;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    ah[r] = nn[tw][r] * rn[r];
                    s.ah[(4 * g + r) * DS + col] = ah[r];
                }
                R.aht[w * TPW + tw][lane] = ah;
                f32x4 zd;
#pragma unroll
                for (int r = 0; r < 4; ++r) zd[r] = -z[tw][r] * rd4[r];
                // B operand at step m: (D^{-1} Z)[4g + m][col] -- held by lane (g, i) as zd[m]
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const f32x4 za = lds4(&s.zt[(16 * q + i) * TS + 4 * g]);
#pragma unroll
                    for (int m = 0; m < 4; ++m) AT[tw][q] = mfma4(za[m], zd[m], AT[tw][q]);
                }
            }
        }
        lds_sync();
        // ---- wave FW: strict(Khat Ahat^T) by column, inverted; wave 1: lower(Qhat Ahat^T)
        if (w == FW) {
            f32x4 km2[2] = {zero4, zero4};
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const f32x4 kr = lds4(&KH[i * DS + 16 * q + 4 * g]);
                const f32x4 ar = lds4(&s.ah[i * DS + 16 * q + 4 * g]);
#pragma unroll
                for (int m = 0; m < 4; ++m) km2[m & 1] = mfma4(kr[m], ar[m], km2[m & 1]);
            }
            const f32x4 km = km2[0] + km2[1];
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
            f32x4 aq2[2] = {zero4, zero4};
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const f32x4 ar = lds4(&s.ah[i * DS + 16 * q + 4 * g]);
                const f32x4 qr = lds4(&QH[i * DS + 16 * q + 4 * g]);
#pragma unroll
                for (int m = 0; m < 4; ++m) aq2[m & 1] = mfma4(ar[m], qr[m], aq2[m & 1]);
            }
            f32x4 aq = aq2[0] + aq2[1];
            // aq lane (g, i): (Ahat Qhat^T)[s = 4g + r][t = i] = (Qhat Ahat^T)[t = i][s = 4g + r]:
            // already the A operand of Y = Aq U; keep s <= t
#pragma unroll
            for (int r = 0; r < 4; ++r) aq[r] = 4 * g + r <= i ? aq[r] : 0.f;
            s.aq[lane] = aq;
        }
        lds_sync();
        // ---- the state step's operands (per tile): Ktil = Tc Khat, Qtil = Qhat - Aq Ktil
        {
            const f32x4 tc = s.top[lane], aqv = s.aq[lane];
            if (tiles) {
#pragma unroll
                for (int tw = 0; tw < TPW; ++tw) {
                    const int col = colof(tw);
                    // B operand at step m: Khat[4g + m][col]
                    f32x4 kb, qb;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        kb[r] = KH[(4 * g + r) * DS + col];
                        qb[r] = QH[(4 * g + r) * DS + col];
                    }
                    f32x4 k0 = mfma4(tc[0], kb[0], zero4), k1 = mfma4(tc[1], kb[1], zero4);
                    k0 = mfma4(tc[2], kb[2], k0);
                    k1 = mfma4(tc[3], kb[3], k1);
                    const f32x4 kt = k0 + k1;  // lane (g, i): Ktil[4g + r][col], the B operand of Aq Ktil
                    f32x4 q0 = qb, q1 = zero4;
                    q0 = mfma4(-aqv[0], kt[0], q0);
                    q1 = mfma4(-aqv[1], kt[1], q1);
                    q0 = mfma4(-aqv[2], kt[2], q0);
                    q1 = mfma4(-aqv[3], kt[3], q1);
                    const f32x4 qt = q0 + q1;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        R.kt[(4 * g + r) * D + col] = kt[r];
                        R.qt[(4 * g + r) * D + col] = qt[r];
                    }
                }
            }
            if (w == 0) R.top[lane] = tc;
            if (w == (TPW > 1 ? FW : NW - 1)) {
                // (Aq Tc)^T = Tc^T Aq^T: A operand Tc^T (lane (g, i) step m:
                // Tc[4g + m][i]), B operand Aq^T (step m: Aq[i][4g + m], the
                // A-order aq); the product lands in Aq Tc's A-operand order
                const float *tf = reinterpret_cast<const float *>(s.top);
                f32x4 a0 = zero4, a1 = zero4;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float tcm = tf[((i >> 2) * 16 + 4 * g + m) * 4 + (i & 3)];
                    if (m & 1) a1 = mfma4(tcm, aqv[m], a1);
                    else a0 = mfma4(tcm, aqv[m], a0);
                }
                R.aqt[lane] = a0 + a1;
            }
        }
        lds_sync();  // chunk tiles free for the next chunk
    }

    if (a.A_out && seg1 == T && tiles) {
#pragma unroll
        for (int tw = 0; tw < TPW; ++tw) {
            const int col = colof(tw);
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                *reinterpret_cast<float4 *>(a.A_out + sb + static_cast<int64_t>(col) * D + 16 * q + 4 * g) =
                    make_float4(AT[tw][q][0], AT[tw][q][1], AT[tw][q][2], AT[tw][q][3]);
        }
    }
}

// Two waves per SIMD: with D = 96's four-wave workgroups, two workgroups per
// compute unit (the other sizes need no more than 256 registers anyway).
template <typename IO, int D>
__global__ __launch_bounds__(64 * alpha_waves<D>()) __attribute__((amdgpu_waves_per_eu(2))) void vla_alpha_kernel(VlaArgs a, const float *__restrict__ Aseg,
                                                                          ChunkRec<D> *__restrict__ rec, int nseg,
                                                                          unsigned int *status) {
    __shared__ AlphaLds<D> s;
    vla_alpha_body<IO, D>(s, a, Aseg, rec, nseg, status);
}

// ================================ state ================================
template <typename IO, int D>
hipError_t launch_d(const VlaArgs &a, hipStream_t stream) {
    const VlaLayout L = vla_layout<D>(a.B, a.T, a.H);
    char *ws = static_cast<char *>(a.ws);
    unsigned int *status = reinterpret_cast<unsigned int *>(ws);
    float *G = reinterpret_cast<float *>(ws + L.g_off);
    float *Aseg = reinterpret_cast<float *>(ws + L.a_off);
    ChunkRec<D> *rec = reinterpret_cast<ChunkRec<D> *>(ws + L.rec_off);
    const int nseg = static_cast<int>(L.nseg);
    const unsigned heads = static_cast<unsigned>(a.B * a.H);
    if (nseg > 1) {
        vla_gram_kernel<IO, D><<<heads * (nseg - 1), 64 * (D / 16), 0, stream>>>(a, G, nseg, status);
        vla_inverse_kernel<D><<<heads * (nseg - 1), 256, 0, stream>>>(a, G, Aseg, nseg);
    }
    vla_alpha_kernel<IO, D><<<heads * nseg, 64 * alpha_waves<D>(), 0, stream>>>(a, Aseg, rec, nseg, status);
    ScanArgs sa{};
    sa.B = a.B;
    sa.T = a.T;
    sa.H = a.H;
    sa.dv = D;
    sa.v = a.v;
    sa.out = a.out;
    sa.S_in = a.S_in;
    sa.S_out = a.S_out;
    sa.side_kind = kSideNone;
    chunk_state_kernel<IO, D, false, false><<<heads * (D / 16), 64 * state_waves<D>(), 0, stream>>>(sa, rec);
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

bool vla_chunked_workspace(const VlaArgs &a, size_t *bytes) {
    VlaLayout L;
    switch (a.d) {
        case 32: L = vla_layout<32>(a.B, a.T, a.H); break;
        case 64: L = vla_layout<64>(a.B, a.T, a.H); break;
        case 96: L = vla_layout<96>(a.B, a.T, a.H); break;
        case 128: L = vla_layout<128>(a.B, a.T, a.H); break;
        default: return false;
    }
    if (a.B * a.H * L.nseg > 0x7fffffff) return false;
    *bytes = L.bytes;
    return true;
}

hipError_t launch_vla_chunked(const VlaArgs &a, hipStream_t stream) {
    if (!vla_chunked_supported(a)) return hipErrorNotSupported;
    return a.dtype == kBF16 ? launch_io<IoBF16>(a, stream) : launch_io<IoF32>(a, stream);
}

}  // namespace lam
