// delta_recurrent.hip -- token-by-token delta-rule scan on gfx950.
//
// The rule ("Mechanisms, trade-offs and cross-layer routing of
// linear-attention architectures", "Technical details"): per token the memory
// is decayed (scalar alpha, or per key channel for Kimi Delta), the residual
// of the decayed memory's prediction along the read key is written along k
// scaled by beta, and the query reads the updated memory.
//
// Schedule.  Rows of W are independent for every variant (row i of the update
// uses only row i of W, v_i / z_i and the shared key), so one chain
// (b, h) is split across workgroups by value rows: each workgroup owns ROWS
// rows of W in registers, TPR lanes per row, each lane CPT = dk/TPR columns
// (interleaved: column = lane_in_row + TPR*m, so LDS reads of the shared key
// and query are conflict-free and broadcast across rows).  Per token one
// fused lane reduction yields W k~, W q~ and k.q, from which
//   r = target - a (W k~),  y = a (W q~) + beta r (k.q),  W = decay W + beta r k^T
// with a = alpha (scalar gates) or folded into k~, q~ (Kimi Delta).
// Tokens stream through LDS in tiles of TT, the next tile prefetched into
// registers while the current one is consumed.  Blocks of one head are placed
// on one XCD so q and k are fetched from HBM once per head.
#include "device_common.h"
#include "lam_internal.h"

namespace lam {
namespace {

constexpr int kThreads = 256;
constexpr int TT = 16;  // tokens per LDS tile

template <int DK>
struct RecShape {
    static constexpr int TPR = DK >= 96 ? 16 : 8;
    static constexpr int CPT = DK / TPR;
    static constexpr int ROWS = kThreads / TPR;
};

template <int VARIANT, typename IO, int DK>
__global__ __launch_bounds__(kThreads) void delta_recurrent_kernel(DeltaArgs a) {
    using Sh = RecShape<DK>;
    constexpr int TPR = Sh::TPR, CPT = Sh::CPT, ROWS = Sh::ROWS;
    constexpr bool kChanDecay = VARIANT == kKimiDelta;
    constexpr bool kScalarDecay = VARIANT == kGatedDeltaNet || VARIANT == kGatedDeltaNet2;
    constexpr bool kGates2 = VARIANT == kGatedDeltaNet2;

    const int T = static_cast<int>(a.T), H = static_cast<int>(a.H), dv = a.dv;
    const int slices = dv / ROWS;
    int head, slice;
    xcd_group_map(blockIdx.x, static_cast<int>(a.B * a.H), slices, head, slice);
    const int b = head / H, h = head % H;

    const int tid = threadIdx.x;
    const int lr = tid % TPR;        // lane within the row group
    const int rl = tid / TPR;        // row within the block
    const int row = slice * ROWS + rl;

    __shared__ float sq[TT][DK], sk[TT][DK];
    __shared__ float sv[TT][ROWS];
    __shared__ float sbeta[TT], salpha[TT];
    __shared__ float sdec[kChanDecay ? TT : 1][kChanDecay ? DK : 1];
    __shared__ float serase[kGates2 ? TT : 1][kGates2 ? DK : 1];
    __shared__ float swrite[kGates2 ? TT : 1][kGates2 ? ROWS : 1];
    __shared__ float sy[TT][ROWS];
    __shared__ float sside[TT][ROWS];  // the routing signal (residual or write value), when asked for
    const bool side = a.side != nullptr;
    const bool side_res = a.side_kind == kSideResidual;

    // ---- memory rows in registers
    float W[CPT];
    const int64_t st_base = ((static_cast<int64_t>(b) * H + h) * dv + row) * DK;
#pragma unroll
    for (int m = 0; m < CPT; ++m) W[m] = a.state_in ? a.state_in[st_base + lr + TPR * m] : 0.f;

    // ---- tile staging: each thread owns fixed slots of the tile
    constexpr int KSLOTS = (TT * DK + kThreads - 1) / kThreads;   // q, k, erase, decay
    constexpr int VSLOTS = (TT * ROWS + kThreads - 1) / kThreads; // v, write
    float rq[KSLOTS], rk[KSLOTS], rdec[kChanDecay ? KSLOTS : 1], rer[kGates2 ? KSLOTS : 1];
    float rv[VSLOTS], rw[kGates2 ? VSLOTS : 1];
    float rbeta = 0.f, ralpha = 1.f;

    auto fetch = [&](int t0) {
#pragma unroll
        for (int s = 0; s < KSLOTS; ++s) {
            const int e = tid + s * kThreads;
            const int t = e / DK, j = e % DK;
            const int tt = t0 + t;
            const bool ok = e < TT * DK && tt < T;
            const int64_t gi = ((static_cast<int64_t>(b) * T + tt) * H + h) * DK + j;
            rq[s] = ok ? IO::ld(a.q, gi) : 0.f;
            rk[s] = ok ? IO::ld(a.k, gi) : 0.f;
            if constexpr (kChanDecay) rdec[s] = ok ? IO::ld(a.alpha, gi) : 1.f;
            if constexpr (kGates2) rer[s] = ok ? IO::ld(a.erase_b, gi) : 0.f;
        }
#pragma unroll
        for (int s = 0; s < VSLOTS; ++s) {
            const int e = tid + s * kThreads;
            const int t = e / ROWS, i = e % ROWS;
            const int tt = t0 + t;
            const bool ok = e < TT * ROWS && tt < T;
            const int64_t gi = ((static_cast<int64_t>(b) * T + tt) * H + h) * dv + slice * ROWS + i;
            rv[s] = ok ? IO::ld(a.v, gi) : 0.f;
            if constexpr (kGates2) rw[s] = ok ? IO::ld(a.write_w, gi) : 0.f;
        }
        if (tid < TT) {
            const int tt = t0 + tid;
            const bool ok = tt < T;
            const int64_t gi = (static_cast<int64_t>(b) * T + tt) * H + h;
            rbeta = ok ? IO::ld(a.beta, gi) : 0.f;
            if constexpr (kScalarDecay) ralpha = ok ? IO::ld(a.alpha, gi) : 1.f;
        }
    };
    auto commit = [&]() {
#pragma unroll
        for (int s = 0; s < KSLOTS; ++s) {
            const int e = tid + s * kThreads;
            if (e < TT * DK) {
                const int t = e / DK, j = e % DK;
                sq[t][j] = rq[s];
                sk[t][j] = rk[s];
                if constexpr (kChanDecay) sdec[t][j] = rdec[s];
                if constexpr (kGates2) serase[t][j] = rer[s];
            }
        }
#pragma unroll
        for (int s = 0; s < VSLOTS; ++s) {
            const int e = tid + s * kThreads;
            if (e < TT * ROWS) {
                const int t = e / ROWS, i = e % ROWS;
                sv[t][i] = rv[s];
                if constexpr (kGates2) swrite[t][i] = rw[s];
            }
        }
        if (tid < TT) {
            sbeta[tid] = rbeta;
            salpha[tid] = ralpha;
        }
    };

    if (T > 0) fetch(0);
    for (int t0 = 0; t0 < T; t0 += TT) {
        __syncthreads();  // previous tile fully consumed (sy stored, LDS free)
        commit();
        __syncthreads();
        if (t0 + TT < T) fetch(t0 + TT);  // overlaps the loads with this tile's math

        const int nt = min(TT, T - t0);
        // Per-token operands of this lane, read one token ahead so the LDS
        // latency overlaps the previous token's update.
        struct Tok {
            float k[CPT], q[CPT], dec[kChanDecay ? CPT : 1], er[kGates2 ? CPT : 1];
            float be, al, target;
        };
        auto load = [&](int t, Tok &o) {
#pragma unroll
            for (int m = 0; m < CPT; ++m) {
                const int j = lr + TPR * m;
                o.k[m] = sk[t][j];
                o.q[m] = sq[t][j];
                if constexpr (kChanDecay) o.dec[m] = sdec[t][j];
                if constexpr (kGates2) o.er[m] = serase[t][j];
            }
            o.be = sbeta[t];
            o.al = kScalarDecay ? salpha[t] : 1.f;
            o.target = sv[t][rl];
            if constexpr (kGates2) o.target *= swrite[t][rl];
        };
        Tok cur, nxt;
        load(0, cur);
        for (int t = 0; t < nt; ++t) {
            if (t + 1 < nt) load(t + 1, nxt);
            float p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
            for (int m = 0; m < CPT; ++m) {
                const float kj = cur.k[m], qj = cur.q[m];
                float rk_ = kj, rq_ = qj;
                if constexpr (kChanDecay) {
                    rk_ = cur.dec[m] * kj;
                    rq_ = cur.dec[m] * qj;
                }
                if constexpr (kGates2) rk_ = cur.er[m] * kj;
                p1 = fmaf(W[m], rk_, p1);
                p2 = fmaf(W[m], rq_, p2);
                p3 = fmaf(kj, qj, p3);
            }
            p1 = group_sum<TPR>(p1);
            p2 = group_sum<TPR>(p2);
            p3 = group_sum<TPR>(p3);
            const float r = cur.target - cur.al * p1;
            const float br = cur.be * r;
            const float y = fmaf(br, p3, cur.al * p2);
#pragma unroll
            for (int m = 0; m < CPT; ++m) {
                const float dec = kChanDecay ? cur.dec[m] : cur.al;
                W[m] = fmaf(br, cur.k[m], dec * W[m]);
            }
            if (lr == 0) {
                sy[t][rl] = y;
                if (side) sside[t][rl] = side_res ? r : cur.target;
            }
            cur = nxt;
        }
        __syncthreads();
        // store the output tile: ROWS contiguous values per token
        for (int e = tid; e < nt * ROWS; e += kThreads) {
            const int t = e / ROWS, i = e % ROWS;
            const int64_t gi = ((static_cast<int64_t>(b) * T + t0 + t) * H + h) * dv + slice * ROWS + i;
            IO::st(a.out, gi, sy[t][i]);
            if (side) IO::st(a.side, gi, sside[t][i]);
        }
    }

    if (a.state_out) {
#pragma unroll
        for (int m = 0; m < CPT; ++m) a.state_out[st_base + lr + TPR * m] = W[m];
    }
}

template <int VARIANT, typename IO>
hipError_t launch_dk(const DeltaArgs &a, hipStream_t stream) {
    auto go = [&](auto kern, int rows) -> hipError_t {
        const int64_t blocks = a.B * a.H * (a.dv / rows);
        kern<<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream>>>(a);
        return hipGetLastError();
    };
    switch (a.dk) {
        case 32: return go(delta_recurrent_kernel<VARIANT, IO, 32>, RecShape<32>::ROWS);
        case 64: return go(delta_recurrent_kernel<VARIANT, IO, 64>, RecShape<64>::ROWS);
        case 96: return go(delta_recurrent_kernel<VARIANT, IO, 96>, RecShape<96>::ROWS);
        case 128: return go(delta_recurrent_kernel<VARIANT, IO, 128>, RecShape<128>::ROWS);
    }
    return hipErrorInvalidValue;
}

template <typename IO>
hipError_t launch_io(const DeltaArgs &a, hipStream_t stream) {
    switch (a.variant) {
        case kDeltaNet: return launch_dk<kDeltaNet, IO>(a, stream);
        case kGatedDeltaNet: return launch_dk<kGatedDeltaNet, IO>(a, stream);
        case kKimiDelta: return launch_dk<kKimiDelta, IO>(a, stream);
        case kGatedDeltaNet2: return launch_dk<kGatedDeltaNet2, IO>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_delta_recurrent(const DeltaArgs &a, hipStream_t stream) {
    return a.dtype == kBF16 ? launch_io<IoBF16>(a, stream) : launch_io<IoF32>(a, stream);
}

}  // namespace lam
