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
//   L  = strict_lower(diag(beta) (E K^T * Gamma))
//   U  = (I + L)^{-1} diag(beta) (Z - diag(gamma) E S^T)
//   Y  = diag(gamma) Q S^T + (lower(Q K^T) * Gamma) U
//   S' = gamma_C S + U^T diag(gamma_C / gamma) K
// Every exponent is g_t - g_s with s <= t (or g_C - g_t), so no factor exceeds
// one and strong decays underflow to zero instead of overflowing.
//
// Schedule.  One workgroup (4 waves) per (b, h, 32-wide slice of dv); rows of
// W are independent, so slices never communicate.  The workgroup walks the
// chunks in order.  Per chunk:
//   staging   q, k (row-major and transposed), v (transposed, fp32) and the
//             gates into LDS from registers prefetched during the previous
//             chunk;
//   prologue  (all waves) wave prefix scan of log a; the lower 16x16 tiles of
//             E K^T and Q K^T on 16x16x32 bf16 MFMA; masks and gates applied
//             in fp32; the four diagonal 16x16 blocks of I + L inverted by
//             forward substitution in fp32;
//   carry     (waves 0 and 1, one 16-column tile of the slice each) E S^T and
//             Q S^T on MFMA, the right-hand side, a blockwise forward solve on
//             16x16x16 MFMA (U_i = D_i (R_i - sum_{j<i} L_ij U_j)), Y, and the
//             state update accumulated straight into the state registers.
// The state slice S^T (dk x 16 per carry wave) lives in MFMA accumulator
// layout for the whole scan.  An accumulator tile holds 4 consecutive rows per
// lane, while a B operand wants 8 consecutive reduction indices; since a
// contraction does not care how its reduction index is ordered, two stacked
// accumulator tiles serve directly as a B operand if the A operand is read
// with the same order (rows 4g..4g+3 and 16+4g..16+4g+3 of each 32-block).
// The same trick feeds U and the right-hand side to the next products without
// an LDS round trip.
#include "device_common.h"
#include "lam_internal.h"

namespace lam {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = 64;    // chunk length (tokens)
constexpr int BV = 32;   // dv columns per workgroup
constexpr int NT = 256;  // threads per workgroup (4 waves)
constexpr int CS = C + 8;  // row stride (elements) of C-wide bf16 LDS tiles
constexpr int DS = 24;     // row stride of the 16x16 diagonal inverses

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x4 bf4(f32x4 x) { return __builtin_convertvector(x, bf16x4); }
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x4 lds4(const __bf16 *p) { return *reinterpret_cast<const bf16x4 *>(p); }

// A operand of a 16x16x32 product from a row-major bf16 LDS matrix: rows
// r0..r0+15, reduction columns c0..c0+31 taken in accumulator order.
__device__ __forceinline__ bf16x8 row_frag(const __bf16 *m, int stride, int r0, int c0, int lane) {
    const __bf16 *p = m + (r0 + (lane & 15)) * stride + c0 + 4 * (lane >> 4);
    return cat8(lds4(p), lds4(p + 16));
}
// A wave-uniform integer the compiler cannot see through (one scalar move).
__device__ __forceinline__ int opaque(int x) {
    int r;
    asm("s_mov_b32 %0, %1" : "=s"(r) : "s"(x));
    return r;
}
// The same fragment read as two independent 8-byte LDS loads.  Each load's
// uniform offset passes through opaque(), so no two loads share a base
// register and the compiler cannot fuse them into ds_read2_b64: on gfx950 a
// conflict-free ds_read_b64 takes about 2 cycles, while ds_read2_b64 of the
// same bytes takes 7.5 (14.8 at these row strides).
typedef __attribute__((address_space(3))) const bf16x4 lds_bf16x4_t;
__device__ __forceinline__ uint32_t lds_address(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void *)p));
}
__device__ __forceinline__ bf16x8 row_frag2(const __bf16 *m, int stride, int r0, int c0, int lane, int) {
    const uint32_t lane_off = 2u * static_cast<uint32_t>((lane & 15) * stride + 4 * (lane >> 4));
    const uint32_t u = lds_address(m) + 2u * static_cast<uint32_t>(r0 * stride + c0);
    const uint32_t a0 = lane_off + static_cast<uint32_t>(opaque(static_cast<int>(u)));
    const uint32_t a1 = lane_off + static_cast<uint32_t>(opaque(static_cast<int>(u + 32u)));
    return cat8(*reinterpret_cast<lds_bf16x4_t *>(static_cast<uintptr_t>(a0)),
                *reinterpret_cast<lds_bf16x4_t *>(static_cast<uintptr_t>(a1)));
}
// Column gather with the gfx950 LDS transpose read.  Within each 16-lane
// group g, lane m supplies the 8-byte piece m[r0 + 4g + m/4][c0 + 4(m%4) ..]
// and lane i receives m[r0 + 4g + j][c0 + i] in slot j = 0..3: four
// consecutive rows of one column, i.e. the accumulator-order operand of a
// reduction over rows, read from a row-major tile.
__device__ __forceinline__ bf16x4 col_gather4(const __bf16 *m, int stride, int r0, int c0, int lane) {
    const int g = lane >> 4, i = lane & 15;
    const __bf16 *p = m + (r0 + 4 * g + (i >> 2)) * stride + c0 + 4 * (i & 3);
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p));
}
// A operand of a 16x16x32 product contracting over rows r0..r0+31 of a
// row-major tile, for output rows = columns c0..c0+15 (accumulator order).
__device__ __forceinline__ bf16x8 col_frag(const __bf16 *m, int stride, int r0, int c0, int lane) {
    return cat8(col_gather4(m, stride, r0, c0, lane), col_gather4(m, stride, r0 + 16, c0, lane));
}
// A operand of a 16x16x16 product: the 16x16 block at (r0, c0).
__device__ __forceinline__ bf16x4 blk_frag(const __bf16 *m, int stride, int r0, int c0, int lane) {
    return lds4(m + (r0 + (lane & 15)) * stride + c0 + 4 * (lane >> 4));
}

struct Raw16 {  // 16 bytes of bf16 from global memory
    uint4 u;
};

template <int VARIANT, int DK>
struct ChunkLds {
    static constexpr bool kGates2 = VARIANT == kGatedDeltaNet2;
    static constexpr int KS = DK + 8;  // row stride of dk-wide bf16 tiles
    alignas(16) __bf16 q[C * KS];
    alignas(16) __bf16 k[C * KS];
    alignas(16) __bf16 e[kGates2 ? C * KS : 8];  // erase-gated keys (Gated DeltaNet-2)
    alignas(16) __bf16 kt[DK * CS];              // keys transposed: [dk][t]
    alignas(16) float vt[BV * (C + 4)];          // value targets transposed: [v][t]
    alignas(16) __bf16 aqk[C * CS];              // lower(Q K^T) * Gamma
    alignas(16) __bf16 ln[C * CS];               // -L (strictly lower blocks used)
    alignas(16) __bf16 dinv[4 * 16 * DS];        // inverses of the diagonal blocks of I + L
    alignas(16) float ld[4 * 16 * 17];           // diagonal blocks of L (fp32)
    alignas(16) float loga[C];
    alignas(16) float beta[C];
    alignas(16) float g[C];
    alignas(16) float gam[C];
    alignas(16) float sc[C];
    alignas(16) __bf16 y[C * (BV + 8)];
};

template <int VARIANT, int DK>
__global__ __launch_bounds__(NT) void delta_chunked_kernel(DeltaArgs a) {
    constexpr bool kGates2 = VARIANT == kGatedDeltaNet2;
    constexpr bool kDecay = VARIANT != kDeltaNet;
    constexpr int KS = DK + 8;
    constexpr int KSTEP = DK / 32;   // 32-wide reduction steps over dk
    constexpr int KT = DK / 16;      // 16-row tiles of S^T
    constexpr int ROW16 = DK / 8;    // 16-byte pieces per dk-row
    constexpr int QK_LOADS = C * ROW16 / NT;
    static_assert(QK_LOADS * NT == C * ROW16, "q/k staging");

    __shared__ ChunkLds<VARIANT, DK> s;

    const int T = static_cast<int>(a.T), H = static_cast<int>(a.H), dv = a.dv;
    const int slices = dv / BV;
    int head, slice;
    xcd_group_map(blockIdx.x, static_cast<int>(a.B * a.H), slices, head, slice);
    const int b = head / H, h = head % H;
    const int v0 = slice * BV;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lg = lane >> 4, lc = lane & 15;

    const uint16_t *gq = static_cast<const uint16_t *>(a.q);
    const uint16_t *gk = static_cast<const uint16_t *>(a.k);
    const uint16_t *gv = static_cast<const uint16_t *>(a.v);
    const uint16_t *geb = static_cast<const uint16_t *>(a.erase_b);
    const uint16_t *gww = static_cast<const uint16_t *>(a.write_w);
    const uint16_t *gal = static_cast<const uint16_t *>(a.alpha);
    const uint16_t *gbe = static_cast<const uint16_t *>(a.beta);
    auto tok = [&](int t) { return (static_cast<int64_t>(b) * T + t) * H + h; };

    // Upper tiles (0,1) and (2,3) of Q K^T enter the 32-wide reduction blocks of
    // the Y product; they are never written, so clear them once.
    for (int i = tid; i < C * CS; i += NT) s.aqk[i] = static_cast<__bf16>(0.f);

    // ---------------------------------------------------------- state
    // Carry waves 0, 1 own S^T[:, 16*wave .. 16*wave+15] as KT accumulator tiles.
    const bool carry = wave < 2;
    f32x4 St[KT];
    {
        const int v = v0 + 16 * (wave & 1) + lc;
        const int64_t base = (static_cast<int64_t>(head) * dv + v) * DK;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            if (carry && a.state_in) {
                const float4 x = *reinterpret_cast<const float4 *>(a.state_in + base + 16 * kt + 4 * lg);
                St[kt] = f32x4{x.x, x.y, x.z, x.w};
            } else {
                St[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }

    // ---------------------------------------------------------- prefetch
    Raw16 rq[QK_LOADS], rk[QK_LOADS], re[kGates2 ? QK_LOADS : 1];
    Raw16 rv, rw;
    float rsc = 0.f;  // thread t < 64: log a_t; 64 <= t < 128: beta_t
    const int nchunks = (T + C - 1) / C;
    auto fetch = [&](int c) {
        const int t0 = c * C;
#pragma unroll
        for (int i = 0; i < QK_LOADS; ++i) {
            const int idx = tid + NT * i, row = idx / ROW16, part = idx % ROW16;
            const bool ok = t0 + row < T;
            const int64_t off = tok(t0 + row) * DK + part * 8;
            rq[i].u = ok ? *reinterpret_cast<const uint4 *>(gq + off) : make_uint4(0, 0, 0, 0);
            rk[i].u = ok ? *reinterpret_cast<const uint4 *>(gk + off) : make_uint4(0, 0, 0, 0);
            if constexpr (kGates2)
                re[i].u = ok ? *reinterpret_cast<const uint4 *>(geb + off) : make_uint4(0, 0, 0, 0);
        }
        {
            const int row = tid >> 2, part = tid & 3;  // 64 rows x 4 pieces of 8
            const bool ok = t0 + row < T;
            const int64_t off = tok(t0 + row) * dv + v0 + part * 8;
            rv.u = ok ? *reinterpret_cast<const uint4 *>(gv + off) : make_uint4(0, 0, 0, 0);
            if constexpr (kGates2)
                rw.u = ok ? *reinterpret_cast<const uint4 *>(gww + off) : make_uint4(0, 0, 0, 0);
        }
        if (tid < 2 * C) {
            const int t = tid & (C - 1);
            const bool ok = t0 + t < T;
            if (tid < C) {
                float la = 0.f;
                if (kDecay && ok) la = fmaxf(logf(bf16_bits_to_f32(gal[tok(t0 + t)])), -150.f);
                rsc = la;
            } else {
                rsc = ok ? bf16_bits_to_f32(gbe[tok(t0 + t)]) : 0.f;
            }
        }
    };
    auto unpack = [](uint32_t w, float &lo, float &hi) {
        lo = __uint_as_float(w << 16);
        hi = __uint_as_float(w & 0xffff0000u);
    };
    auto commit = [&]() {
#pragma unroll
        for (int i = 0; i < QK_LOADS; ++i) {
            const int idx = tid + NT * i, row = idx / ROW16, part = idx % ROW16;
            *reinterpret_cast<uint4 *>(&s.q[row * KS + part * 8]) = rq[i].u;
            *reinterpret_cast<uint4 *>(&s.k[row * KS + part * 8]) = rk[i].u;
            const uint32_t kw[4] = {rk[i].u.x, rk[i].u.y, rk[i].u.z, rk[i].u.w};
            uint16_t *ktp = reinterpret_cast<uint16_t *>(s.kt);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                ktp[(part * 8 + 2 * j) * CS + row] = static_cast<uint16_t>(kw[j] & 0xffffu);
                ktp[(part * 8 + 2 * j + 1) * CS + row] = static_cast<uint16_t>(kw[j] >> 16);
            }
            if constexpr (kGates2) {
                const uint32_t bw[4] = {re[i].u.x, re[i].u.y, re[i].u.z, re[i].u.w};
                uint32_t ew[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float k0, k1, b0, b1;
                    unpack(kw[j], k0, k1);
                    unpack(bw[j], b0, b1);
                    ew[j] = static_cast<uint32_t>(f32_to_bf16_bits(k0 * b0)) |
                            (static_cast<uint32_t>(f32_to_bf16_bits(k1 * b1)) << 16);
                }
                *reinterpret_cast<uint4 *>(&s.e[row * KS + part * 8]) = make_uint4(ew[0], ew[1], ew[2], ew[3]);
            }
        }
        {
            const int row = tid >> 2, part = tid & 3;
            const uint32_t vw[4] = {rv.u.x, rv.u.y, rv.u.z, rv.u.w};
            const uint32_t ww[4] = {rw.u.x, rw.u.y, rw.u.z, rw.u.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float x0, x1;
                unpack(vw[j], x0, x1);
                if constexpr (kGates2) {
                    float w0, w1;
                    unpack(ww[j], w0, w1);
                    x0 *= w0;
                    x1 *= w1;
                }
                s.vt[(part * 8 + 2 * j) * (C + 4) + row] = x0;
                s.vt[(part * 8 + 2 * j + 1) * (C + 4) + row] = x1;
            }
        }
        if (tid < C)
            s.loga[tid] = rsc;
        else if (tid < 2 * C)
            s.beta[tid - C] = rsc;
    };

    if (nchunks > 0) fetch(0);
    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * C;
        const int nvalid = min(C, T - t0);
        __syncthreads();  // LDS of the previous chunk is no longer read
        commit();
        __syncthreads();
        if (c + 1 < nchunks) fetch(c + 1);

        // ---- gate prefix scan (wave 0): g, gamma = exp(g), sc = exp(g_C - g)
        if (wave == 0) {
            float x = s.loga[lane];
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const float y = __shfl_up(x, o, 64);
                if (lane >= o) x += y;
            }
            const float gl = __shfl(x, 63, 64);
            s.g[lane] = x;
            s.gam[lane] = expf(x);
            s.sc[lane] = expf(gl - x);
        }
        __syncthreads();

        // ---- lower tiles of E K^T (-> L) and Q K^T (-> Aqk), 20 tiles over 4 waves
        for (int job = wave; job < 20; job += 4) {
            const bool isqk = job >= 10;
            int jj = isqk ? job - 10 : job, ti = 0;
            while (jj > ti) { jj -= ti + 1; ++ti; }
            const int si = jj;
            const __bf16 *am = isqk ? s.q : (kGates2 ? s.e : s.k);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < KSTEP; ++p)
                acc = mfma32(row_frag(am, KS, 16 * ti, 32 * p, lane), row_frag(s.k, KS, 16 * si, 32 * p, lane), acc);
            const int scol = 16 * si + lc;
            const float gs = s.g[scol];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * ti + 4 * lg + r;
                const float gm = expf(fminf(s.g[t] - gs, 0.f));
                if (isqk) {
                    const float val = scol <= t ? acc[r] * gm : 0.f;
                    s.aqk[t * CS + scol] = static_cast<__bf16>(val);
                } else {
                    const float val = scol < t ? s.beta[t] * gm * acc[r] : 0.f;
                    if (ti == si)
                        s.ld[(ti * 16 + (t & 15)) * 17 + lc] = val;
                    else
                        s.ln[t * CS + scol] = static_cast<__bf16>(-val);
                }
            }
        }
        __syncthreads();

        // ---- inverses of the diagonal blocks of I + L (wave w: block w; lane = column)
        if (lane < 16) {
            const float *L = &s.ld[wave * 16 * 17];
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = i == lane ? 1.f : 0.f;
#pragma unroll
            for (int i = 1; i < 16; ++i) {
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < i; ++m) acc = fmaf(L[i * 17 + m], x[m], acc);
                if (i > lane) x[i] = -acc;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) s.dinv[(wave * 16 + i) * DS + lane] = static_cast<__bf16>(x[i]);
        }
        __syncthreads();

        // ---- carry (waves 0, 1)
        if (carry) {
            const int vt = wave;  // 16-column tile within the slice
            bf16x8 bS[KSTEP];
#pragma unroll
            for (int p = 0; p < KSTEP; ++p) bS[p] = cat8(bf4(St[2 * p]), bf4(St[2 * p + 1]));
            const __bf16 *em = kGates2 ? s.e : s.k;
            f32x4 rhs[4], y[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                f32x4 kp = {0.f, 0.f, 0.f, 0.f}, qp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < KSTEP; ++p) {
                    kp = mfma32(row_frag(em, KS, 16 * ti, 32 * p, lane), bS[p], kp);
                    qp = mfma32(row_frag(s.q, KS, 16 * ti, 32 * p, lane), bS[p], qp);
                }
                const int t = 16 * ti + 4 * lg;
                const float4 z = *reinterpret_cast<const float4 *>(&s.vt[(16 * vt + lc) * (C + 4) + t]);
                const float zz[4] = {z.x, z.y, z.z, z.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    rhs[ti][r] = s.beta[t + r] * fmaf(-s.gam[t + r], kp[r], zz[r]);
                    y[ti][r] = s.gam[t + r] * qp[r];
                }
            }
            // blockwise forward solve: U_i = D_i (R_i - sum_{j<i} L_ij U_j)
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            f32x4 u[4];
            bf16x4 ub[4];
            u[0] = mfma16(blk_frag(s.dinv, DS, 0, 0, lane), bf4(rhs[0]), zero);
            ub[0] = bf4(u[0]);
#pragma unroll
            for (int i = 1; i < 4; ++i) {
                f32x4 x = rhs[i];
#pragma unroll
                for (int j = 0; j < i; ++j) x = mfma16(blk_frag(s.ln, CS, 16 * i, 16 * j, lane), ub[j], x);
                u[i] = mfma16(blk_frag(s.dinv, DS, 16 * i, 0, lane), bf4(x), zero);
                ub[i] = bf4(u[i]);
            }
            // Y = gamma Q S^T + lower(Q K^T * Gamma) U
            const bf16x8 bU0 = cat8(ub[0], ub[1]), bU1 = cat8(ub[2], ub[3]);
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                y[ti] = mfma32(row_frag(s.aqk, CS, 16 * ti, 0, lane), bU0, y[ti]);
                if (ti >= 2) y[ti] = mfma32(row_frag(s.aqk, CS, 16 * ti, 32, lane), bU1, y[ti]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    s.y[(16 * ti + 4 * lg + r) * (BV + 8) + 16 * vt + lc] = static_cast<__bf16>(y[ti][r]);
            }
            // S^T = gamma_C S^T + K^T diag(gamma_C / gamma) U
            f32x4 us[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int r = 0; r < 4; ++r) us[ti][r] = u[ti][r] * s.sc[16 * ti + 4 * lg + r];
            const bf16x8 bW0 = cat8(bf4(us[0]), bf4(us[1])), bW1 = cat8(bf4(us[2]), bf4(us[3]));
            const float gC = s.gam[C - 1];
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                f32x4 acc = St[kt] * gC;
                acc = mfma32(row_frag(s.kt, CS, 16 * kt, 0, lane), bW0, acc);
                acc = mfma32(row_frag(s.kt, CS, 16 * kt, 32, lane), bW1, acc);
                St[kt] = acc;
            }
        }
        __syncthreads();

        // ---- store the output tile (nvalid rows x 32 columns)
        {
            const int row = tid >> 2, part = tid & 3;
            if (row < nvalid) {
                const uint4 x = *reinterpret_cast<const uint4 *>(&s.y[row * (BV + 8) + part * 8]);
                *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.out) + tok(t0 + row) * dv + v0 + part * 8) = x;
            }
        }
    }

    if (carry && a.state_out) {
        const int v = v0 + 16 * wave + lc;
        const int64_t base = (static_cast<int64_t>(head) * dv + v) * DK;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
            *reinterpret_cast<float4 *>(a.state_out + base + 16 * kt + 4 * lg) =
                make_float4(St[kt][0], St[kt][1], St[kt][2], St[kt][3]);
    }
}

// ===========================================================================
// Pipelined schedule (DeltaNet, Gated DeltaNet): 8 waves per workgroup, two
// per SIMD, in three roles.
//   carry  (waves 0-1, one 16-column tile of the slice each): the critical
//          path E S^T -> right-hand side -> blockwise solve -> state update;
//          U is published to LDS as soon as the solve ends.
//   output (waves 2-3, same tiles): Q S^T while the carry solves, then Y from
//          the published U, the output store, and a replica of the state
//          update (the same MFMA sequence on the same operands, so the two
//          copies of the state stay bit-identical without a state handoff).
//   producers (waves 4-7): stage chunk c+1 into the other half of a
//          double-buffered LDS set and compute its state-independent
//          matrices, a quarter each.
// All eight waves meet at one LDS barrier per chunk.  Producers order their
// staging writes before their tile reads, and each output wave waits for its
// carry wave's U, through bounded LDS counters.  Only producers issue global
// loads (two chunks ahead), so carry waves never wait on HBM.
// ===========================================================================
constexpr int NLB = 6;     // strictly lower 16x16 blocks of a 64-row chunk
constexpr int NT8 = 512;   // threads per workgroup of the pipelined schedule

template <int DK>
struct PipeLds {
    static constexpr int KS = DK + 8;
    static constexpr int VS = BV + 8;
    struct Raw {  // staged token streams of one chunk
        alignas(16) __bf16 q[C * KS];
        alignas(16) __bf16 k[C * KS];
        alignas(16) __bf16 v[C * VS];    // the workgroup's value columns
        alignas(16) float la[C];         // log2 of the decay (0 for padding)
        alignas(16) float beta[C];
    };
    struct Der {  // state-independent matrices of one chunk
        alignas(16) __bf16 aqk[C * CS];          // lower(Q K^T) * Gamma
        alignas(16) __bf16 lnb[NLB * 16 * DS];   // -L, strictly lower blocks
        alignas(16) __bf16 dinv[4 * 16 * DS];    // (I + L_ii)^{-1}
        alignas(16) float gam[C];                // gamma_t
        alignas(16) float sc[C];                 // gamma_C / gamma_t
        alignas(16) float beta[C];
    };
    Raw raw[2];
    Der der[2];
    alignas(16) float ld[4 * 16 * 20]; // diagonal blocks of L, fp32, stored by column: [block][col][row]
    alignas(16) float gw[4][C];        // per-producer copy of the gate prefix sums
    alignas(16) __bf16 ys[2][C * 24];  // output staging, one 64x16 tile per output wave
    alignas(16) bf16x4 uh[2][4][64];   // U of the current chunk, per tile, fragment order
    alignas(16) bf16x4 sh[2][2][DK / 16][64];  // bf16 state fragments: [parity][tile][16-row block]
    unsigned int pcount;               // producer arrivals
    unsigned int ucount[2];            // U publications per tile
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier that orders LDS only: outstanding global loads (the
// producers' prefetch) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts (fixed order of additions, so it is bitwise reproducible).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_shift(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, true));
}
__device__ __forceinline__ float wave_prefix_sum(float x) {
    x += dpp_shift<0x111, 0xf>(x);  // row_shr:1
    x += dpp_shift<0x112, 0xf>(x);  // row_shr:2
    x += dpp_shift<0x114, 0xf>(x);  // row_shr:4
    x += dpp_shift<0x118, 0xf>(x);  // row_shr:8
    x += dpp_shift<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
    x += dpp_shift<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

// Value of lane n of this lane's 16-lane row (DPP row_newbcast).
template <int N>
__device__ __forceinline__ float row_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + N, 0xf, 0xf, false));
}

// Column c of (I + L)^{-1} for a unit lower-triangular 16x16 block whose
// strictly lower part L arrives by columns: lane c of a 16-lane row holds
// column c (lcol[i] = L[i][c]).  Forward substitution x_i = -sum_{m<i}
// L[i][m] x_m, with L[i][m] broadcast from lane m of the row, in fp32.
template <int M = 0>
__device__ __forceinline__ void fsub_terms(float &acc, const float (&lcol)[16], const float (&x)[16], int i) {
    if constexpr (M < 15) {
        if (M < i) acc = fmaf(row_bcast<M>(lcol[i]), x[M], acc);
        fsub_terms<M + 1>(acc, lcol, x, i);
    }
}
__device__ __forceinline__ void unit_lower_inverse_column(const float (&lcol)[16], float (&x)[16], int c) {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = i == c ? 1.f : 0.f;
#pragma unroll
    for (int i = 1; i < 16; ++i) {
        float acc = 0.f;
        fsub_terms(acc, lcol, x, i);
        if (i > c) x[i] = -acc;
    }
}

// Publish: make this wave's LDS writes visible, then count one arrival.
__device__ __forceinline__ void lds_arrive(unsigned int *cnt, int lane) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0) __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Bounded wait until `*cnt` reaches `target`.  Every wave leaves the loop
// after at most 2^22 polls, so a lost arrival can slow the kernel down but
// never hang it.
__device__ __forceinline__ void lds_wait(unsigned int *cnt, unsigned int target) {
    for (int it = 0; it < (1 << 22); ++it) {
        if (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) break;
        __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// S^T = gamma_C S^T + K^T diag(gamma_C / gamma) U for one 16-column tile,
// shared by the carry wave and its output-wave replica.
template <int KT, typename Raw, typename Der>
__device__ __forceinline__ void state_update(f32x4 (&St)[KT], const Raw &R, const Der &D, const bf16x4 (&ub)[4],
                                             int KS, int lane) {
    const int lg = lane >> 4;
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
    for (int h2 = 0; h2 < 2; ++h2) {
        const bf16x8 bW = h2 ? bW1 : bW0;
        bf16x8 af[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) af[kt] = col_frag(R.k, KS, 32 * h2, 16 * kt, lane);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) St[kt] = mfma32(af[kt], bW, St[kt]);
    }
}

// Lower tiles of Q K^T computed by producers 2 and 3.
struct QkTilesLow {
    static constexpr int n = 6;
    static constexpr int ti[6] = {0, 1, 1, 2, 2, 2}, si[6] = {0, 0, 1, 0, 1, 2};
};
struct QkTilesRow3 {
    static constexpr int n = 4;
    static constexpr int ti[4] = {3, 3, 3, 3}, si[4] = {0, 1, 2, 3};
};

template <int VARIANT, int DK>
__global__ __launch_bounds__(NT8) void delta_chunked_pipe_kernel(DeltaArgs a) {
    constexpr bool kDecay = VARIANT != kDeltaNet;
    constexpr int KS = DK + 8;
    constexpr int KSTEP = DK / 32;
    constexpr int KT = DK / 16;
    using Lds = PipeLds<DK>;
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
    // 16, from an argument the compiler cannot constant-fold (T >= 0 always)
    const int sixteen = __builtin_amdgcn_readfirstlane(16 + (a.T < 0 ? 1 : 0));

    for (int i = tid; i < C * CS; i += NT8) {
        s.der[0].aqk[i] = static_cast<__bf16>(0.f);
        s.der[1].aqk[i] = static_cast<__bf16>(0.f);
    }
    if (tid == 0) {
        s.pcount = 0u;
        s.ucount[0] = s.ucount[1] = 0u;
    }
    __syncthreads();  // counters and cleared tiles visible before any role starts

    if (wave < 4) {
        // ========================= carry and output ==========================
        const bool is_carry = wave < 2;
        const int vt = wave & 1;
        f32x4 St[KT];
        const int vcol = v0 + 16 * vt + lc;
        const int64_t sbase = (static_cast<int64_t>(head) * dv + vcol) * DK;
        // carry: publish the bf16 B-operand fragments of S^T for chunk `c`
        auto publish_state = [&](int c) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) s.sh[c & 1][vt][kt][lane] = bf4(St[kt]);
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
            publish_state(0);
        }
        lds_barrier();  // chunk 0 staged and derived, initial state published
        for (int c = 0; c < nchunks; ++c) {
            const typename Lds::Raw &R = s.raw[c & 1];
            const typename Lds::Der &D = s.der[c & 1];
            bf16x8 bS[KSTEP];
            if (is_carry) {
#pragma unroll
                for (int p = 0; p < KSTEP; ++p) bS[p] = cat8(bf4(St[2 * p]), bf4(St[2 * p + 1]));
            } else {
#pragma unroll
                for (int p = 0; p < KSTEP; ++p)
                    bS[p] = cat8(s.sh[c & 1][vt][2 * p][lane], s.sh[c & 1][vt][2 * p + 1][lane]);
            }
            // E S^T (carry) or Q S^T (output), four row tiles
            const __bf16 *am = is_carry ? R.k : R.q;
            f32x4 xp[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) xp[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < KSTEP; ++p) {
                bf16x8 af[4];
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) af[ti] = row_frag2(am, KS, 16 * ti, 32 * p, lane, sixteen);
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) xp[ti] = mfma32(af[ti], bS[p], xp[ti]);
            }
            if (is_carry) {
                f32x4 rhs[4];
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
                    const int t = 16 * ti + 4 * lg;
                    const bf16x4 z = col_gather4(R.v, Lds::VS, 16 * ti, 16 * vt, lane);
                    const float4 be = *reinterpret_cast<const float4 *>(&D.beta[t]);
                    const float4 ga = *reinterpret_cast<const float4 *>(&D.gam[t]);
                    const float bb[4] = {be.x, be.y, be.z, be.w}, gg[4] = {ga.x, ga.y, ga.z, ga.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) rhs[ti][r] = bb[r] * fmaf(-gg[r], xp[ti][r], static_cast<float>(z[r]));
                }
                // blockwise forward solve U_i = D_i (R_i - sum_{j<i} L_ij U_j)
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                bf16x4 ub[4];
                ub[0] = bf4(mfma16(blk_frag(D.dinv, DS, 0, 0, lane), bf4(rhs[0]), zero));
#pragma unroll
                for (int i = 1; i < 4; ++i) {
                    f32x4 x = rhs[i];
#pragma unroll
                    for (int j = 0; j < i; ++j)
                        x = mfma16(blk_frag(D.lnb, DS, 16 * (i * (i - 1) / 2 + j), 0, lane), ub[j], x);
                    ub[i] = bf4(mfma16(blk_frag(D.dinv, DS, 16 * i, 0, lane), bf4(x), zero));
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) s.uh[vt][i][lane] = ub[i];
                lds_arrive(&s.ucount[vt], lane);
                state_update<KT>(St, R, D, ub, KS, lane);
                if (c + 1 < nchunks) publish_state(c + 1);
            } else {
                lds_wait(&s.ucount[vt], static_cast<unsigned int>(c + 1));
                bf16x4 ub[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) ub[i] = s.uh[vt][i][lane];
                // Y = gamma Q S^T + lower(Q K^T * Gamma) U
                f32x4 y[4];
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
                    const float4 ga = *reinterpret_cast<const float4 *>(&D.gam[16 * ti + 4 * lg]);
                    y[ti] = xp[ti] * f32x4{ga.x, ga.y, ga.z, ga.w};
                }
                const bf16x8 bU0 = cat8(ub[0], ub[1]), bU1 = cat8(ub[2], ub[3]);
                bf16x8 yf[6];
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) yf[ti] = row_frag2(D.aqk, CS, 16 * ti, 0, lane, sixteen);
                yf[4] = row_frag2(D.aqk, CS, 32, 32, lane, sixteen);
                yf[5] = row_frag2(D.aqk, CS, 48, 32, lane, sixteen);
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) y[ti] = mfma32(yf[ti], bU0, y[ti]);
                y[2] = mfma32(yf[4], bU1, y[2]);
                y[3] = mfma32(yf[5], bU1, y[3]);
                __bf16 *ys = s.ys[vt];
#pragma unroll
                for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                    for (int r = 0; r < 4; ++r) ys[(16 * ti + 4 * lg + r) * 24 + lc] = static_cast<__bf16>(y[ti][r]);
                const int t0 = c * C;
                if (t0 + lane < T) {  // each lane stores one 32-byte output row segment
                    const uint2 *src = reinterpret_cast<const uint2 *>(&ys[lane * 24]);
                    uint2 *dst = reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + tok(t0 + lane) * dv + v0 + 16 * vt);
#pragma unroll
                    for (int i = 0; i < 4; ++i) dst[i] = src[i];
                }
            }
            lds_barrier();
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
        const uint16_t *gsc = static_cast<const uint16_t *>(pw == 0 ? a.alpha : a.beta);
        // Coalesced staging: a dk-wide bf16 row is DK/8 16-byte pieces, so
        // one load instruction covers 64*8/DK consecutive rows; a row of the
        // workgroup's 32 value columns is 4 pieces (16 rows per instruction).
        constexpr int PPR = DK / 8;             // 16-byte pieces per q/k row
        constexpr int RPI = 64 / PPR;           // rows per load instruction
        constexpr int NQK = 16 / RPI;           // instructions per producer per stream
        uint4 rq[NQK], rk[NQK], rv;
        uint32_t rs = 0u;    // raw bf16 bits of the decay (pw 0) or beta (pw 1) of row `lane`
        uint32_t okm = 0u;   // bit i: row of q/k load i inside the sequence; bit NQK: v row; bit NQK+1: gate row
        // Loads read clamped, always valid rows; rows past the end are replaced
        // by padding at commit, so no loaded value is consumed here and the
        // loads stay in flight until the next chunk's staging.
        auto fetch = [&](int c) {
            const int t0 = c * C;
            okm = 0u;
#pragma unroll
            for (int i = 0; i < NQK; ++i) {
                const int t = t0 + 16 * pw + RPI * i + lane / PPR;
                okm |= (t < T ? 1u : 0u) << i;
                const int64_t o = tok(min(t, T - 1)) * DK + (lane % PPR) * 8;
                rq[i] = *reinterpret_cast<const uint4 *>(gq + o);
                rk[i] = *reinterpret_cast<const uint4 *>(gk + o);
            }
            {
                const int t = t0 + 16 * pw + (lane >> 2);
                okm |= (t < T ? 1u : 0u) << NQK;
                rv = *reinterpret_cast<const uint4 *>(gv + tok(min(t, T - 1)) * dv + v0 + 8 * (lane & 3));
            }
            if (pw <= 1) {
                const int t = t0 + lane;
                okm |= (t < T ? 1u : 0u) << (NQK + 1);
                if (pw == 1 || kDecay) rs = static_cast<uint32_t>(gsc[tok(min(t, T - 1))]);
            }
        };
        // rows past the end become zeros (a bitwise mask keeps the registers
        // out of the select-of-aggregates form that lands them in scratch)
        auto masked = [](uint4 x, uint32_t m) { return make_uint4(x.x & m, x.y & m, x.z & m, x.w & m); };
        auto commit = [&](int c) {
            typename Lds::Raw &R = s.raw[c & 1];
#pragma unroll
            for (int i = 0; i < NQK; ++i) {
                const int row = 16 * pw + RPI * i + lane / PPR;
                const uint32_t m = 0u - ((okm >> i) & 1u);
                *reinterpret_cast<uint4 *>(&R.q[row * KS + (lane % PPR) * 8]) = masked(rq[i], m);
                *reinterpret_cast<uint4 *>(&R.k[row * KS + (lane % PPR) * 8]) = masked(rk[i], m);
            }
            {
                const int row = 16 * pw + (lane >> 2);
                *reinterpret_cast<uint4 *>(&R.v[row * Lds::VS + 8 * (lane & 3)]) = masked(rv, 0u - ((okm >> NQK) & 1u));
            }
            const bool gok = (okm >> (NQK + 1)) & 1u;
            if (pw == 0) {
                const float al = bf16_bits_to_f32(static_cast<uint16_t>(rs));
                R.la[lane] = (kDecay && gok) ? fmaxf(__builtin_amdgcn_logf(al), -200.f) : 0.f;
            } else if (pw == 1) {
                R.beta[lane] = gok ? bf16_bits_to_f32(static_cast<uint16_t>(rs)) : 0.f;
            }
        };
        // State-independent matrices of chunk c, a quarter per producer.
        auto derive = [&](int c) {
            const typename Lds::Raw &R = s.raw[c & 1];
            typename Lds::Der &D = s.der[c & 1];
            const float g = wave_prefix_sum(R.la[lane]);  // every producer keeps its own copy
            float *gw = s.gw[pw];
            gw[lane] = g;
            float gt[4][4], bt[4][4], gs[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                const float4 g4 = *reinterpret_cast<const float4 *>(&gw[16 * ti + 4 * lg]);
                const float4 b4 = *reinterpret_cast<const float4 *>(&R.beta[16 * ti + 4 * lg]);
                gt[ti][0] = g4.x; gt[ti][1] = g4.y; gt[ti][2] = g4.z; gt[ti][3] = g4.w;
                bt[ti][0] = b4.x; bt[ti][1] = b4.y; bt[ti][2] = b4.z; bt[ti][3] = b4.w;
                gs[ti] = gw[16 * ti + lc];
            }
            if (pw == 0) {
                // gates, diagonal tiles of E K^T -> L_ii (fp32), their inverses
                const float gl = __shfl(g, 63, 64);
                D.gam[lane] = exp2_fast(g);
                D.sc[lane] = exp2_fast(gl - g);
                D.beta[lane] = R.beta[lane];
                f32x4 acc[4];
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) acc[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < KSTEP; ++p) {
                    bf16x8 kf[4];
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti) kf[ti] = row_frag2(R.k, KS, 16 * ti, 32 * p, lane, sixteen);
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti) acc[ti] = mfma32(kf[ti], kf[ti], acc[ti]);
                }
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
                    float val[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int tr = 4 * lg + r;
                        val[r] = lc < tr ? bt[ti][r] * exp2_fast(gt[ti][r] - gs[ti]) * acc[ti][r] : 0.f;
                    }
                    float *dst = &s.ld[(ti * 16 + lc) * 20 + 4 * lg];  // column lc, rows 4lg..4lg+3
                    *reinterpret_cast<float2 *>(dst) = make_float2(val[0], val[1]);
                    *reinterpret_cast<float2 *>(dst + 2) = make_float2(val[2], val[3]);
                }
                // inverses of the diagonal blocks: lane = (block lg, column lc)
                float lcol[16], x[16];
                const float *src = &s.ld[(lg * 16 + lc) * 20];
#pragma unroll
                for (int i = 0; i < 16; i += 2) {
                    const float2 v2 = *reinterpret_cast<const float2 *>(src + i);
                    lcol[i] = v2.x;
                    lcol[i + 1] = v2.y;
                }
                unit_lower_inverse_column(lcol, x, lc);
#pragma unroll
                for (int i = 0; i < 16; ++i) D.dinv[(16 * lg + i) * DS + lc] = static_cast<__bf16>(x[i]);
            } else if (pw == 1) {
                // strictly lower off-diagonal tiles of E K^T -> -L blocks
                constexpr int TI[NLB] = {1, 2, 2, 3, 3, 3}, SI[NLB] = {0, 0, 1, 0, 1, 2};
                f32x4 acc[NLB];
#pragma unroll
                for (int j = 0; j < NLB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < KSTEP; ++p) {
                    bf16x8 kf[4];
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti) kf[ti] = row_frag2(R.k, KS, 16 * ti, 32 * p, lane, sixteen);
#pragma unroll
                    for (int j = 0; j < NLB; ++j) acc[j] = mfma32(kf[TI[j]], kf[SI[j]], acc[j]);
                }
#pragma unroll
                for (int j = 0; j < NLB; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        D.lnb[(16 * j + 4 * lg + r) * DS + lc] = static_cast<__bf16>(
                            -(bt[TI[j]][r] * exp2_fast(gt[TI[j]][r] - gs[SI[j]]) * acc[j][r]));
            } else {
                // lower tiles of Q K^T -> Aqk: rows 0-2 (6 tiles) or row 3 (4 tiles)
                auto qk_tiles = [&](auto tiles) {
                    constexpr int NJ = decltype(tiles)::n;
                    f32x4 acc[NJ];
#pragma unroll
                    for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int p = 0; p < KSTEP; ++p) {
                        bf16x8 kf[4], qf[4];
#pragma unroll
                        for (int ti = 0; ti < 4; ++ti) {
                            kf[ti] = row_frag2(R.k, KS, 16 * ti, 32 * p, lane, sixteen);
                            qf[ti] = row_frag2(R.q, KS, 16 * ti, 32 * p, lane, sixteen);
                        }
#pragma unroll
                        for (int j = 0; j < NJ; ++j) acc[j] = mfma32(qf[tiles.ti[j]], kf[tiles.si[j]], acc[j]);
                    }
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        const int ti = tiles.ti[j], si = tiles.si[j];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int tr = 4 * lg + r;
                            const float val = (si < ti || lc <= tr) ? acc[j][r] * exp2_fast(gt[ti][r] - gs[si]) : 0.f;
                            D.aqk[(16 * ti + tr) * CS + 16 * si + lc] = static_cast<__bf16>(val);
                        }
                    }
                };
                if (pw == 2)
                    qk_tiles(QkTilesLow{});
                else
                    qk_tiles(QkTilesRow3{});
            }
        };

        unsigned int target = 0;
        if (nchunks > 0) {
            fetch(0);
            commit(0);
            target += 4;
            lds_arrive(&s.pcount, lane);
            lds_wait(&s.pcount, target);
            if (nchunks > 1) fetch(1);
            derive(0);
        }
        lds_barrier();  // chunk 0 staged and derived
        for (int c = 0; c < nchunks; ++c) {
            if (c + 1 < nchunks) {
                commit(c + 1);
                target += 4;
                lds_arrive(&s.pcount, lane);
                lds_wait(&s.pcount, target);
                if (c + 2 < nchunks) fetch(c + 2);
                derive(c + 1);
            }
            lds_barrier();
        }
    }
}

template <int VARIANT>
hipError_t launch_var(const DeltaArgs &a, hipStream_t stream) {
    const unsigned blocks = static_cast<unsigned>(a.B * a.H * (a.dv / BV));
    constexpr bool kPipe = VARIANT != kGatedDeltaNet2;
    switch (a.dk) {
        case 64:
            if constexpr (kPipe) delta_chunked_pipe_kernel<VARIANT, 64><<<blocks, NT8, 0, stream>>>(a);
            else delta_chunked_kernel<VARIANT, 64><<<blocks, NT, 0, stream>>>(a);
            break;
        case 128:
            if constexpr (kPipe) delta_chunked_pipe_kernel<VARIANT, 128><<<blocks, NT8, 0, stream>>>(a);
            else delta_chunked_kernel<VARIANT, 128><<<blocks, NT, 0, stream>>>(a);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool delta_chunked_supported(const DeltaArgs &a) {
    return a.dtype == kBF16 && a.variant != kKimiDelta && (a.dk == 64 || a.dk == 128) &&
           a.dv % BV == 0;
}

hipError_t launch_delta_chunked(const DeltaArgs &a, hipStream_t stream) {
    if (!delta_chunked_supported(a)) return hipErrorNotSupported;
    switch (a.variant) {
        case kDeltaNet: return launch_var<kDeltaNet>(a, stream);
        case kGatedDeltaNet: return launch_var<kGatedDeltaNet>(a, stream);
        case kGatedDeltaNet2: return launch_var<kGatedDeltaNet2>(a, stream);
    }
    return hipErrorNotSupported;
}

}  // namespace lam
