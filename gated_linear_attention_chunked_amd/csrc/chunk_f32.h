// chunk_f32.h -- the fp32 chunked scan shared by VLA and by the fp32 form of
// the delta-rule family (DeltaNet, Gated DeltaNet, Gated DeltaNet-2).
//
// Both rules, cut into chunks of VC = 16 tokens (rows = tokens, S the memory
// at the chunk start), take one state step of the same shape once the
// state-independent parts of a chunk are formed:
//   U = Tc V - Ktil S^T,   Y = Qtil S^T + (Aq Tc) V,   S^T <- gC S^T + Ahat^T U.
// VLA ("Technical summary: Variational Linear Attention (VLA)", section 2.3):
//   Tc = (I + strict(Khat Ahat^T))^{-1}, Ktil = Tc Khat, Aq = lower(Qhat Ahat^T),
//   Qtil = Qhat - Aq Ktil, Ahat the gates, gC = 1.
// The delta rule ("Mechanisms, trade-offs and cross-layer routing of
// linear-attention architectures", "Technical details"), in the residual
// form with gamma_t the running decay and Gamma_ts = gamma_t / gamma_s:
//   Tc = (I + strict(E K^T * Gamma) diag(beta))^{-1}, Ktil = Tc diag(gamma) E,
//   Aq = lower(Q K^T * Gamma) diag(beta), Qtil = diag(gamma) Q - Aq Ktil,
//   Ahat = diag(beta gamma_C / gamma) K, gC = gamma_C,
// so U is the chunk's residuals (Z - decayed prediction), V the targets z.
// A derivation kernel per rule writes these operands to a per-chunk record;
// the state kernel below runs the step.
#pragma once

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
// Workgroup barrier that orders LDS only.  Threads of these kernels share
// data only through LDS, and a plain __syncthreads() would also wait for
// every global load in flight (the next chunks' prefetch) at each barrier.
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// f(icst<0>) ... f(icst<N - 1>)
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &f) {
    if constexpr (I < N) {
        f(icst<I>{});
        static_for<N, I + 1>(f);
    }
}
// f(icst<0>) ... f(icst<14>)
template <int I = 0, typename F>
__device__ __forceinline__ void static_for15(F &f) {
    if constexpr (I < 15) {
        f(icst<I>{});
        static_for15<I + 1>(f);
    }
}

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



// Per-chunk record the derivation writes for the state kernel (DK = the key
// dimension; rows past the end of the sequence are zero).
template <int DK>
struct ChunkRec {
    float kt[VC * DK];        // Ktil, rows t
    float qt[VC * DK];        // Qtil, rows t
    f32x4 aht[DK / 16][64];   // Ahat^T tiles, A-operand order: lane (g, i) of tile j holds Ahat[4g + m][16j + i]
    f32x4 top[64];            // Tc, A-operand order
    f32x4 aqt[64];            // Aq Tc, A-operand order
    f32x4 gc;                 // gC (the chunk's decay of the state) in every slot; unused without decay
};

// What the state kernel reads and writes besides the records.
struct ScanArgs {
    int64_t B, T, H;
    int dv;                  // value width DV (a multiple of 16)
    const void *v, *w;       // targets [B,T,H,DV]; write gates (z = w * v) or NULL
    void *out;               // y [B,T,H,DV]
    const float *S_in;       // [B,H,DV,DK] fp32 or NULL (zero)
    float *S_out;            // [B,H,DV,DK] fp32 or NULL
    void *side;              // per-token routing signal [B,T,H,DV] or NULL
    int side_kind;           // kSideResidual (U) or kSideValue (z)
    // the backward pass's forward recompute (KEEP) also writes:
    float *s_chunks;         // S^T at the start of every even chunk, [B*H][pairs][DK][DV] fp32
    float *u_f32;            // the residuals U, [B,T,H,DV] fp32
};

// Key tiles of S^T per carry wave of the state kernel: one at DK = 32, two
// from DK = 64 on, so a workgroup has at most four carries (one per SIMD) and,
// at about 240 registers a lane, two workgroups share a CU.
template <int DK>
__host__ __device__ constexpr int state_tpw() { return DK >= 64 ? 2 : 1; }
template <int DK>
__host__ __device__ constexpr int state_carries() { return DK / 16 / state_tpw<DK>(); }
// With fewer than four carries one more wave forms the output and Tc V on the
// free SIMD; with four, carry 3 forms the output and carry 2 Tc V.
template <int DK>
__host__ __device__ constexpr int state_waves() { return state_carries<DK>() < 4 ? state_carries<DK>() + 1 : 4; }
template <int DK>
__host__ __device__ constexpr int state_y_wave() { return state_carries<DK>() < 4 ? state_carries<DK>() : 3; }
template <int DK>
__host__ __device__ constexpr int state_v_wave() { return state_carries<DK>() < 4 ? state_carries<DK>() : 2; }

// One workgroup per (b, h, 16 value rows of S).  Carry wave w keeps the TPW
// 16 x 16 tiles of S^T at key rows 16 (TPW w + j) .. + 15 and the workgroup's
// value columns; the products over the key dimension are summed across the
// waves through LDS (fixed order, so every wave forms the same sums).
// DECAY: the records carry gC; GATES2: the targets are z = w * v; KEEP:
// also the state at every chunk start and U in fp32 (the backward pass's
// forward recompute).
template <typename IO, int DK, bool DECAY, bool GATES2, bool KEEP = false>
__global__ __launch_bounds__(64 * state_waves<DK>()) void chunk_state_kernel(ScanArgs a,
                                                                             const ChunkRec<DK> *__restrict__ rec) {
    constexpr int TPW = state_tpw<DK>();
    constexpr int NW = state_carries<DK>();
    constexpr int YW = state_y_wave<DK>();  // the wave that forms the output
    constexpr int VW = state_v_wave<DK>();  // the wave that forms Tc V
    __shared__ f32x4 part[2][2][NW][64];  // [chunk parity][Ktil S^T, Qtil S^T][wave][lane]
    __shared__ f32x4 tv[2][64];           // [chunk parity] Tc V
    const int T = static_cast<int>(a.T), H = static_cast<int>(a.H);
    int head, vt;
    const int DV = a.dv;
    xcd_group_map(blockIdx.x, static_cast<int>(a.B * a.H), DV / 16, head, vt);
    const int b = head / H, h = head % H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, i = lane & 15;
    const int vcol = 16 * vt + i;
    const int64_t sb = static_cast<int64_t>(head) * DV * DK;
    const int nch = (T + VC - 1) / VC;
    // Token rows of the value-shaped tensors: a wave-uniform element offset of
    // (b, t0, h, column 16 vt) plus a 32-bit lane offset (row 4g + r of the
    // chunk, column i); H * DV is at most 2^24, so the lane offsets fit.
    const int HD = H * DV;
    const int64_t cbase = (static_cast<int64_t>(b) * T * H + h) * DV + 16 * vt;
    auto chunk_base = [&](int t0) { return cbase + static_cast<int64_t>(t0) * HD; };
    int roff[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) roff[r] = (4 * g + r) * HD + i;

    // ST[j] lane (g, i): S^T[kr + 4g + r][vcol] = S[vcol][kr + 4g + r], kr = 16 (TPW w + j)
    f32x4 ST[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
        ST[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (a.S_in && w < NW) {
            const float4 x = *reinterpret_cast<const float4 *>(a.S_in + sb + static_cast<int64_t>(vcol) * DK +
                                                               16 * (TPW * w + j) + 4 * g);
            ST[j] = f32x4{x.x, x.y, x.z, x.w};
        }
    }
    const ChunkRec<DK> *R0 = rec + static_cast<int64_t>(head) * nch;
    // KEEP forms no output: no Qtil or Aq Tc operands, no Y products
    const bool is_carry = w < NW, is_y = !KEEP && w == YW;
    constexpr int QN = KEEP ? 1 : TPW;
    struct Ops {
        f32x4 kt[TPW], qt[QN], aht[TPW], top, aqt;
        float v[4], w[GATES2 ? 4 : 1], gc;
    };
    // Every wave issues the same loads whatever its role (an output-only wave
    // reads the last carry's operands and ignores them): with role-dependent
    // loads the compiler's load-counter waits would drain the whole ring.
    const int wc = min(w, NW - 1);
    auto load = [&](int c, Ops &o) {  // past the end: the last chunk again (never used)
        const int cc = min(c, nch - 1);
        const ChunkRec<DK> &R = R0[cc];
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int kr = 16 * (TPW * wc + j);
            o.kt[j] = *reinterpret_cast<const f32x4 *>(&R.kt[i * DK + kr + 4 * g]);
            if constexpr (!KEEP) o.qt[j] = *reinterpret_cast<const f32x4 *>(&R.qt[i * DK + kr + 4 * g]);
            o.aht[j] = R.aht[TPW * wc + j][lane];
        }
        if constexpr (!KEEP) o.aqt = R.aqt[lane];
        o.top = R.top[lane];
        const int t0 = cc * VC, n = min(VC, T - t0);
        const int64_t cb = chunk_base(t0);
        const int last = (n - 1) * HD + i;  // rows past the end read the chunk's last row
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int off = 4 * g + r < n ? roff[r] : last;
            o.v[r] = IO::ld(a.v, cb + off);
            if constexpr (GATES2) o.w[r] = IO::ld(a.w, cb + off);
        }
        o.gc = DECAY ? R.gc[0] : 1.f;
    };
    // rows 4g + r < n of a chunk's output (branch-free for whole chunks)
    auto store_rows = [&](void *dst, int64_t cb, int n, const f32x4 &x) {
        if (n == VC) {
#pragma unroll
            for (int r = 0; r < 4; ++r) IO::st(dst, cb + roff[r], x[r]);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (4 * g + r < n) IO::st(dst, cb + roff[r], x[r]);
        }
    };
    // one chunk's step from its operand set
    auto step = [&](const Ops &cur, int c) {
        const int p = c & 1, t0 = c * VC, n = min(VC, T - t0);
        const int64_t cb = chunk_base(t0);
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        if (KEEP && is_carry && (c & 1) == 0) {  // the state at this pair of chunks' start, S^T rows
            float *dst = a.s_chunks + (static_cast<int64_t>(head) * ((nch + 1) / 2) + (c >> 1)) * DK * DV + vcol;
#pragma unroll
            for (int j = 0; j < TPW; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[static_cast<int64_t>(16 * (TPW * w + j) + 4 * g + r) * DV] = ST[j][r];
        }
        if (is_carry) {
            // partial Ktil S^T and Qtil S^T over this wave's key rows (two
            // accumulators per product keep the dependent chains short)
            f32x4 pk0 = zero, pk1 = zero, pq0 = zero, pq1 = zero;
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                pk0 = mfma4(cur.kt[j][0], ST[j][0], pk0);
                pk1 = mfma4(cur.kt[j][1], ST[j][1], pk1);
                if constexpr (!KEEP) {
                    pq0 = mfma4(cur.qt[j][0], ST[j][0], pq0);
                    pq1 = mfma4(cur.qt[j][1], ST[j][1], pq1);
                }
                pk0 = mfma4(cur.kt[j][2], ST[j][2], pk0);
                pk1 = mfma4(cur.kt[j][3], ST[j][3], pk1);
                if constexpr (!KEEP) {
                    pq0 = mfma4(cur.qt[j][2], ST[j][2], pq0);
                    pq1 = mfma4(cur.qt[j][3], ST[j][3], pq1);
                }
            }
            part[p][0][w][lane] = pk0 + pk1;
            if constexpr (!KEEP) part[p][1][w][lane] = pq0 + pq1;
        }
        // V's rows (zero past the end), the B operand of Tc V and (Aq Tc) V
        f32x4 vb;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float z = GATES2 ? cur.v[r] * cur.w[r] : cur.v[r];
            vb[r] = 4 * g + r < n ? z : 0.f;
        }
        if (w == VW) {
            f32x4 a0 = mfma4(cur.top[0], vb[0], zero), a1 = mfma4(cur.top[1], vb[1], zero);
            a0 = mfma4(cur.top[2], vb[2], a0);
            a1 = mfma4(cur.top[3], vb[3], a1);
            tv[p][lane] = a0 + a1;
        }
        f32x4 y0 = zero;
        if (!KEEP && is_y) {
            f32x4 y1 = mfma4(cur.aqt[1], vb[1], zero);
            y0 = mfma4(cur.aqt[0], vb[0], zero);
            y1 = mfma4(cur.aqt[3], vb[3], y1);
            y0 = mfma4(cur.aqt[2], vb[2], y0);
            y0 += y1;
        }
        lds_sync();
        if (is_carry) {
            // U = Tc V - Ktil S^T (rows past the end: zero), summed in a fixed
            // order so every wave forms the same U; then S^T += Ahat^T U
            f32x4 z = part[p][0][0][lane];
#pragma unroll
            for (int j = 1; j < NW; ++j) z += part[p][0][j][lane];
            const f32x4 u = tv[p][lane] - z;
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                f32x4 d0 = mfma4(cur.aht[j][0], u[0], zero), d1 = mfma4(cur.aht[j][1], u[1], zero);
                d0 = mfma4(cur.aht[j][2], u[2], d0);
                d1 = mfma4(cur.aht[j][3], u[3], d1);
                if constexpr (DECAY) ST[j] = ST[j] * cur.gc + (d0 + d1);
                else ST[j] += d0 + d1;
            }
            if (a.side_kind == kSideResidual && w == 0) store_rows(a.side, cb, n, u);  // the residuals U
            if (KEEP && w == 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (4 * g + r < n) a.u_f32[cb + roff[r]] = u[r];
            }
        }
        if (!KEEP && is_y) {  // Y = Qtil S^T + (Aq Tc) V
            f32x4 y = part[p][1][0][lane];
#pragma unroll
            for (int j = 1; j < NW; ++j) y += part[p][1][j][lane];
            y += y0;
            if (a.out) store_rows(a.out, cb, n, y);
            if (a.side_kind == kSideValue) store_rows(a.side, cb, n, vb);  // the write values z
        }
    };
    // A ring of NS operand sets: the loads run NS chunks ahead (the records
    // come from L2 or HBM, a step takes about a microsecond); every trip
    // refills each set it consumes (past the end: the last chunk again,
    // never used), so the loads in flight always form the same queue.  Three
    // sets keep the kernel under 256 registers a lane, so two four-wave
    // workgroups share a CU (two with KEEP's extra stores).
    constexpr int NS = KEEP ? 2 : 3;
    Ops o[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) load(j, o[j]);
    int c = 0;
    for (; c + NS <= nch; c += NS) {
        auto trip = [&](auto jc) {
            constexpr int j = decltype(jc)::value;
            step(o[j], c + j);
            load(c + j + NS, o[j]);
        };
        static_for<NS>(trip);
    }
    auto tail = [&](auto jc) {
        constexpr int j = decltype(jc)::value;
        if (c + j < nch) step(o[j], c + j);
    };
    static_for<NS>(tail);
    if (a.S_out && is_carry) {
#pragma unroll
        for (int j = 0; j < TPW; ++j)
            *reinterpret_cast<float4 *>(a.S_out + sb + static_cast<int64_t>(vcol) * DK + 16 * (TPW * w + j) + 4 * g) =
                make_float4(ST[j][0], ST[j][1], ST[j][2], ST[j][3]);
    }
}



// ------------------------------------------------------------ adjoint scan
// Reverse mode of the state step above (the delta-rule form, Ktil =
// Tc diag(gamma) E).  With G' = dL/dS^T at a chunk's end, G the same at its
// start and dY the chunk's output cotangents, the adjoint of
//   U = Tc Z - Ktil S^T,  Y = diag(gamma) Q S^T + Aq U,  S'^T = gC S^T + Ahat^T U
// is, per chunk in reverse,
//   dX = Tc^T (Aq^T dY + Ahat G'^T) = (Aq Tc)^T dY + Ahat' G'^T,  Ahat' = Tc^T Ahat,
//   G  = gC G' + (diag(gamma) Q)^T dY - (diag(gamma) E)^T dX,
// and dX is the gradient of the chunk's targets Z.  It has the state step's
// shape: one product over the key dimension (Ahat' G'^T) summed across the
// waves, a state-independent term ((Aq Tc)^T dY) formed beside it, and a
// rank-16 update of the carried tiles.  Ahat' and the transposed operands
// come from the same derivation, in this record.
template <int DK>
struct AdjRec {
    float ap[VC * DK];          // Ahat' = Tc^T Ahat, rows t
    f32x4 gqt[DK / 16][64];     // (diag(gamma) Q)^T tiles: lane (g, i) of tile j holds gamma_{4g+m} Q[4g + m][16j + i]
    f32x4 get[DK / 16][64];     // (diag(gamma) E)^T tiles, the same order
    f32x4 aqtt[64];             // (Aq Tc)^T, A-operand order
    f32x4 gc;                   // gC in every slot; unused without decay
};

struct AdjArgs {
    int64_t B, T, H;
    int dv;                      // value width DV (a multiple of 16)
    const void *dy;              // output cotangents [B,T,H,DV], storage dtype
    const void *v, *w;           // targets and write gates (Gated DeltaNet-2), else NULL
    const float *dS_in;          // cotangent of the final state [B,H,DV,DK] or NULL (zero)
    float *dS_out;               // cotangent of the initial state [B,H,DV,DK] or NULL
    float *ds_chunks;            // G' at the end of every pair of chunks (odd chunks, and the
                                 // last chunk), the layout of s_chunks
    float *dx;                   // dX [B,T,H,DV] fp32
    float *dv_out, *dw_out;      // gradients of v and (Gated DeltaNet-2) w, [B,T,H,DV] fp32
};

// One workgroup per (b, h, 16 value columns), chunks in reverse; roles as
// in chunk_state_kernel (carry waves hold TPW tiles of G^T, the wave VW
// forms the state-independent term).
template <typename IO, int DK, bool DECAY, bool GATES2>
__global__ __launch_bounds__(64 * state_waves<DK>()) void chunk_adjoint_kernel(AdjArgs a,
                                                                               const AdjRec<DK> *__restrict__ rec) {
    constexpr int TPW = state_tpw<DK>();
    constexpr int NW = state_carries<DK>();
    constexpr int VW = state_v_wave<DK>();
    __shared__ f32x4 part[2][NW][64];  // [step parity][wave][lane]: Ahat' G' partials
    __shared__ f32x4 tv[2][64];        // [step parity] (Aq Tc)^T dY
    const int T = static_cast<int>(a.T), H = static_cast<int>(a.H);
    int head, vt;
    const int DV = a.dv;
    xcd_group_map(blockIdx.x, static_cast<int>(a.B * a.H), DV / 16, head, vt);
    const int b = head / H, h = head % H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, i = lane & 15;
    const int vcol = 16 * vt + i;
    const int64_t sb = static_cast<int64_t>(head) * DV * DK;
    const int nch = (T + VC - 1) / VC;
    const int HD = H * DV;
    const int64_t cbase = (static_cast<int64_t>(b) * T * H + h) * DV + 16 * vt;
    auto chunk_base = [&](int t0) { return cbase + static_cast<int64_t>(t0) * HD; };
    int roff[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) roff[r] = (4 * g + r) * HD + i;

    // GT[j] lane (g, i): G^T[kr + 4g + r][vcol], kr = 16 (TPW w + j)
    f32x4 GT[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
        GT[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (a.dS_in && w < NW) {
            const float4 x = *reinterpret_cast<const float4 *>(a.dS_in + sb + static_cast<int64_t>(vcol) * DK +
                                                               16 * (TPW * w + j) + 4 * g);
            GT[j] = f32x4{x.x, x.y, x.z, x.w};
        }
    }
    const AdjRec<DK> *R0 = rec + static_cast<int64_t>(head) * nch;
    const bool is_carry = w < NW;
    struct Ops {
        f32x4 ap[TPW], gq[TPW], ge[TPW], aq;
        float y[4], v[GATES2 ? 4 : 1], w[GATES2 ? 4 : 1], gc;
    };
    const int wc = min(w, NW - 1);
    // step s works on chunk nch - 1 - s; past the end: chunk 0 again (never used)
    auto load = [&](int st, Ops &o) {
        const int cc = max(nch - 1 - st, 0);
        const AdjRec<DK> &R = R0[cc];
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int kr = 16 * (TPW * wc + j);
            o.ap[j] = *reinterpret_cast<const f32x4 *>(&R.ap[i * DK + kr + 4 * g]);
            o.gq[j] = R.gqt[TPW * wc + j][lane];
            o.ge[j] = R.get[TPW * wc + j][lane];
        }
        o.aq = R.aqtt[lane];
        const int t0 = cc * VC, n = min(VC, T - t0);
        const int64_t cb = chunk_base(t0);
        const int last = (n - 1) * HD + i;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int off = 4 * g + r < n ? roff[r] : last;
            o.y[r] = IO::ld(a.dy, cb + off);
            if constexpr (GATES2) {
                o.v[r] = IO::ld(a.v, cb + off);
                o.w[r] = IO::ld(a.w, cb + off);
            }
        }
        o.gc = DECAY ? R.gc[0] : 1.f;
    };
    auto step = [&](const Ops &cur, int st) {
        const int c = nch - 1 - st, p = st & 1, t0 = c * VC, n = min(VC, T - t0);
        const int64_t cb = chunk_base(t0);
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        if (is_carry) {
            // G' (the cotangent of the state after this chunk) at the end of
            // each pair of chunks, kept for the gradient kernel
            if ((c & 1) || c == nch - 1) {
                float *dst = a.ds_chunks + (static_cast<int64_t>(head) * ((nch + 1) / 2) + (c >> 1)) * DK * DV + vcol;
#pragma unroll
                for (int j = 0; j < TPW; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) dst[static_cast<int64_t>(16 * (TPW * w + j) + 4 * g + r) * DV] = GT[j][r];
            }
            // partial Ahat' G' over this wave's key rows
            f32x4 pk0 = zero, pk1 = zero;
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                pk0 = mfma4(cur.ap[j][0], GT[j][0], pk0);
                pk1 = mfma4(cur.ap[j][1], GT[j][1], pk1);
                pk0 = mfma4(cur.ap[j][2], GT[j][2], pk0);
                pk1 = mfma4(cur.ap[j][3], GT[j][3], pk1);
            }
            part[p][w][lane] = pk0 + pk1;
        }
        // dY's rows (zero past the end): the B operand of (Aq Tc)^T dY and of the update
        f32x4 yb;
#pragma unroll
        for (int r = 0; r < 4; ++r) yb[r] = 4 * g + r < n ? cur.y[r] : 0.f;
        if (w == VW) {
            f32x4 a0 = mfma4(cur.aq[0], yb[0], zero), a1 = mfma4(cur.aq[1], yb[1], zero);
            a0 = mfma4(cur.aq[2], yb[2], a0);
            a1 = mfma4(cur.aq[3], yb[3], a1);
            tv[p][lane] = a0 + a1;
        }
        lds_sync();
        if (is_carry) {
            // dX = (Aq Tc)^T dY + Ahat' G' (summed in a fixed order), then
            // G^T <- gC G^T + (gamma Q)^T dY - (gamma E)^T dX
            f32x4 z = part[p][0][lane];
#pragma unroll
            for (int j = 1; j < NW; ++j) z += part[p][j][lane];
            const f32x4 dx = tv[p][lane] + z;
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                f32x4 d0 = mfma4(cur.gq[j][0], yb[0], zero), d1 = mfma4(cur.gq[j][1], yb[1], zero);
                d0 = mfma4(cur.gq[j][2], yb[2], d0);
                d1 = mfma4(cur.gq[j][3], yb[3], d1);
                d0 = mfma4(cur.ge[j][0], -dx[0], d0);
                d1 = mfma4(cur.ge[j][1], -dx[1], d1);
                d0 = mfma4(cur.ge[j][2], -dx[2], d0);
                d1 = mfma4(cur.ge[j][3], -dx[3], d1);
                if constexpr (DECAY) GT[j] = GT[j] * cur.gc + (d0 + d1);
                else GT[j] += d0 + d1;
            }
            if (w == 0) {  // dX, and the gradients of the targets z = w * v (z = v)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (4 * g + r < n) {
                        const int64_t o = cb + roff[r];
                        a.dx[o] = dx[r];
                        if constexpr (GATES2) {
                            a.dv_out[o] = cur.w[r] * dx[r];
                            a.dw_out[o] = cur.v[r] * dx[r];
                        } else {
                            a.dv_out[o] = dx[r];
                        }
                    }
                }
            }
        }
    };
    constexpr int NS = 3;
    Ops o[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) load(j, o[j]);
    int st = 0;
    for (; st + NS <= nch; st += NS) {
        auto trip = [&](auto jc) {
            constexpr int j = decltype(jc)::value;
            step(o[j], st + j);
            load(st + j + NS, o[j]);
        };
        static_for<NS>(trip);
    }
    auto tail = [&](auto jc) {
        constexpr int j = decltype(jc)::value;
        if (st + j < nch) step(o[j], st + j);
    };
    static_for<NS>(tail);
    if (a.dS_out && is_carry) {
#pragma unroll
        for (int j = 0; j < TPW; ++j)
            *reinterpret_cast<float4 *>(a.dS_out + sb + static_cast<int64_t>(vcol) * DK + 16 * (TPW * w + j) + 4 * g) =
                make_float4(GT[j][0], GT[j][1], GT[j][2], GT[j][3]);
    }
}

}  // namespace
}  // namespace lam
