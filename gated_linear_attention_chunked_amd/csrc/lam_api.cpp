// lam_api.cpp -- the C ABI declared in include/lam.h: argument validation
// (host only, before any HIP call) and dispatch to the kernel launchers.
#include "lam.h"

#include <limits.h>
#include <stdint.h>

#include "lam_internal.h"

namespace {

bool supported_head(int64_t d) { return d == 32 || d == 64 || d == 96 || d == 128; }

// a * b without overflow past 2^62; false on overflow or negative operands.
bool mul_ok(int64_t a, int64_t b, int64_t &r) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > (INT64_C(1) << 62) / a) return false;
    r = a * b;
    return true;
}

bool elems(int64_t B, int64_t T, int64_t H, int64_t n, int64_t &r) {
    int64_t x;
    return mul_ok(B, T, x) && mul_ok(x, H, x) && mul_ok(x, n, r);
}

bool overlaps(const void *a, int64_t abytes, const void *b, int64_t bbytes) {
    if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + static_cast<uintptr_t>(bbytes) && b0 < a0 + static_cast<uintptr_t>(abytes);
}

lam_status from_hip(hipError_t e) { return e == hipSuccess ? LAM_OK : LAM_ERR_HIP; }

// Token-row offsets inside a chunk (up to 64 rows of H * d elements) are
// formed in 32 bits by the kernels.
constexpr int64_t kMaxRowElems = INT64_C(1) << 24;

enum Schedule { kNone, kRecurrent, kChunked };

// Shape, enum and size checks shared by lam_forward and its workspace query.
lam_status check_delta_shape(int variant, int dtype, int64_t B, int64_t T, int64_t H, int64_t dk,
                             int64_t dv, int algo) {
    if (variant < LAM_DELTANET || variant > LAM_GATED_DELTANET2) return LAM_ERR_INVALID_ARG;
    if (dtype != LAM_F32 && dtype != LAM_BF16) return LAM_ERR_INVALID_ARG;
    if (algo < LAM_ALGO_AUTO || algo > LAM_ALGO_CHUNKED) return LAM_ERR_INVALID_ARG;
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return LAM_ERR_INVALID_ARG;
    if (!supported_head(dk) || !supported_head(dv)) return LAM_ERR_UNSUPPORTED;
    int64_t nk, nv, ns, nst;
    if (!elems(B, T, H, dk, nk) || !elems(B, T, H, dv, nv) || !elems(B, T, H, 1, ns) ||
        !elems(B, 1, H, dk * dv, nst))
        return LAM_ERR_INVALID_ARG;
    // grid size and 32-bit in-chain indices
    if (B * H > (INT64_C(1) << 24) || T > INT_MAX / 2) return LAM_ERR_INVALID_ARG;
    if (H * (dk > dv ? dk : dv) > kMaxRowElems) return LAM_ERR_INVALID_ARG;
    return LAM_OK;
}

// The schedule a validated call runs and the workspace it needs.
lam_status plan_delta(const lam::DeltaArgs &a, int algo, Schedule *sched, size_t *ws) {
    *ws = 0;
    *sched = kNone;
    if (a.B == 0 || a.H == 0) return LAM_OK;
    const bool chunked_ok = lam::delta_chunked_supported(a);
    if (algo == LAM_ALGO_CHUNKED && !chunked_ok) return LAM_ERR_UNSUPPORTED;
    if (a.T == 0) {  // nothing to scan: the initial state is copied (recurrent kernel)
        *sched = kRecurrent;
        return LAM_OK;
    }
    if (algo == LAM_ALGO_RECURRENT || !chunked_ok) {
        *sched = kRecurrent;
        return LAM_OK;
    }
    if (!lam::delta_chunked_workspace(a, ws)) return LAM_ERR_INVALID_ARG;
    *sched = kChunked;
    return LAM_OK;
}

lam::DeltaArgs shape_args(int variant, int dtype, int64_t B, int64_t T, int64_t H, int64_t dk,
                          int64_t dv) {
    lam::DeltaArgs a{};
    a.variant = variant;
    a.dtype = dtype;
    a.B = B;
    a.T = T;
    a.H = H;
    a.dk = static_cast<int>(dk);
    a.dv = static_cast<int>(dv);
    return a;
}

lam_status check_vla_shape(int dtype, int64_t B, int64_t T, int64_t H, int64_t d, int algo) {
    if (dtype != LAM_F32 && dtype != LAM_BF16) return LAM_ERR_INVALID_ARG;
    if (algo < LAM_ALGO_AUTO || algo > LAM_ALGO_CHUNKED) return LAM_ERR_INVALID_ARG;
    if (B < 0 || T < 0 || H < 0 || d <= 0) return LAM_ERR_INVALID_ARG;
    if (!supported_head(d)) return LAM_ERR_UNSUPPORTED;
    int64_t n, nst;
    if (!elems(B, T, H, d, n) || !elems(B, 1, H, d * d, nst)) return LAM_ERR_INVALID_ARG;
    if (B * H > (INT64_C(1) << 24) || T > INT_MAX / 2) return LAM_ERR_INVALID_ARG;
    if (H * d > kMaxRowElems) return LAM_ERR_INVALID_ARG;
    return LAM_OK;
}

lam_status plan_vla(const lam::VlaArgs &a, int algo, Schedule *sched, size_t *ws) {
    *ws = 0;
    *sched = kNone;
    if (a.B == 0 || a.H == 0) return LAM_OK;
    const bool chunked_ok = lam::vla_chunked_supported(a);
    if (algo == LAM_ALGO_CHUNKED && !chunked_ok) return LAM_ERR_UNSUPPORTED;
    if (a.T == 0 || algo == LAM_ALGO_RECURRENT || !chunked_ok) {
        *sched = kRecurrent;
        return LAM_OK;
    }
    if (!lam::vla_chunked_workspace(a, ws)) return LAM_ERR_INVALID_ARG;
    *sched = kChunked;
    return LAM_OK;
}

// The workspace a call needs: present, large enough, aligned, and clear of
// every other argument.
bool workspace_ok(const void *ws, size_t have, size_t need, const void *const *args,
                  const int64_t *arg_bytes, int nargs) {
    if (need == 0) return true;
    if (!ws || have < need || reinterpret_cast<uintptr_t>(ws) % 256 != 0) return false;
    if (need > static_cast<size_t>(INT64_MAX)) return false;
    for (int i = 0; i < nargs; ++i)
        if (overlaps(ws, static_cast<int64_t>(need), args[i], arg_bytes[i])) return false;
    return true;
}

}  // namespace

extern "C" {

const char *lam_status_string(int s) {
    switch (s) {
        case LAM_OK: return "ok";
        case LAM_ERR_INVALID_ARG: return "invalid argument";
        case LAM_ERR_UNSUPPORTED: return "unsupported shape, dtype or algorithm";
        case LAM_ERR_HIP: return "HIP launch failure";
        case LAM_ERR_SCRATCH_LIMIT: return "call needs more workspace than the no-allocation scratch holds";
    }
    return "unknown status";
}

int lam_abi_version(void) { return 201; }

int lam_select_algo(int variant, int dtype, int64_t T, int64_t dk, int64_t dv) {
    if (variant < LAM_DELTANET || variant > LAM_GATED_DELTANET2) return -1;
    if (dtype != LAM_F32 && dtype != LAM_BF16) return -1;
    if (T < 0 || !supported_head(dk) || !supported_head(dv)) return -1;
    lam::DeltaArgs a{};
    a.variant = variant;
    a.dtype = dtype;
    a.B = 1;
    a.T = T;
    a.H = 1;
    a.dk = static_cast<int>(dk);
    a.dv = static_cast<int>(dv);
    return (T > 0 && lam::delta_chunked_supported(a)) ? LAM_ALGO_CHUNKED : LAM_ALGO_RECURRENT;
}

lam_status lam_forward_workspace_size(int variant, int dtype, int64_t B, int64_t T, int64_t H,
                                      int64_t dk, int64_t dv, int algo, size_t *bytes) {
    if (!bytes) return LAM_ERR_INVALID_ARG;
    *bytes = 0;
    lam_status st = check_delta_shape(variant, dtype, B, T, H, dk, dv, algo);
    if (st != LAM_OK) return st;
    Schedule sched;
    return plan_delta(shape_args(variant, dtype, B, T, H, dk, dv), algo, &sched, bytes);
}

lam_status lam_forward(int variant, int dtype, int64_t B, int64_t T, int64_t H, int64_t dk,
                       int64_t dv, const void *q, const void *k, const void *v,
                       const void *alpha, const void *erase_b, const void *write_w,
                       const void *beta, const float *state_in, void *out, float *state_out,
                       void *workspace, size_t workspace_bytes, int algo, hipStream_t stream) {
    return lam_forward_side(variant, dtype, B, T, H, dk, dv, q, k, v, alpha, erase_b, write_w, beta,
                            state_in, out, state_out, LAM_SIDE_NONE, nullptr, workspace,
                            workspace_bytes, algo, stream);
}

lam_status lam_forward_side(int variant, int dtype, int64_t B, int64_t T, int64_t H, int64_t dk,
                            int64_t dv, const void *q, const void *k, const void *v,
                            const void *alpha, const void *erase_b, const void *write_w,
                            const void *beta, const float *state_in, void *out, float *state_out,
                            int side, void *side_out, void *workspace, size_t workspace_bytes,
                            int algo, hipStream_t stream) {
    lam_status st = check_delta_shape(variant, dtype, B, T, H, dk, dv, algo);
    if (st != LAM_OK) return st;
    if (side < LAM_SIDE_NONE || side > LAM_SIDE_VALUE) return LAM_ERR_INVALID_ARG;
    if (side == LAM_SIDE_NONE) side_out = nullptr;
    if (B == 0 || H == 0) return LAM_OK;
    int64_t nk, nv, ns, nst;
    elems(B, T, H, dk, nk);
    elems(B, T, H, dv, nv);
    elems(B, T, H, 1, ns);
    elems(B, 1, H, dk * dv, nst);
    if (T > 0) {
        if (!q || !k || !v || !beta || !out) return LAM_ERR_INVALID_ARG;
        if (variant != LAM_DELTANET && !alpha) return LAM_ERR_INVALID_ARG;
        if (variant == LAM_GATED_DELTANET2 && (!erase_b || !write_w)) return LAM_ERR_INVALID_ARG;
        if (side != LAM_SIDE_NONE && !side_out) return LAM_ERR_INVALID_ARG;
    }
    const int64_t es = dtype == LAM_BF16 ? 2 : 4;
    const int64_t out_bytes = nv * es;
    if (side_out) {  // the side output may overlap nothing else
        const void *other[] = {q, k, v, variant == LAM_DELTANET ? nullptr : alpha,
                               variant == LAM_GATED_DELTANET2 ? erase_b : nullptr,
                               variant == LAM_GATED_DELTANET2 ? write_w : nullptr, beta, state_in,
                               out, state_out};
        const int64_t ob[] = {nk * es, nk * es, nv * es, (variant == LAM_KIMI_DELTA ? nk : ns) * es,
                              nk * es, nv * es, ns * es, nst * 4, out_bytes, nst * 4};
        for (int i = 0; i < 10; ++i)
            if (overlaps(side_out, out_bytes, other[i], ob[i])) return LAM_ERR_INVALID_ARG;
    }
    const int64_t alpha_bytes = (variant == LAM_KIMI_DELTA ? nk : ns) * es;
    if (overlaps(out, out_bytes, q, nk * es) || overlaps(out, out_bytes, k, nk * es) ||
        overlaps(out, out_bytes, v, nv * es) || overlaps(out, out_bytes, beta, ns * es) ||
        (variant != LAM_DELTANET && overlaps(out, out_bytes, alpha, alpha_bytes)) ||
        (variant == LAM_GATED_DELTANET2 && (overlaps(out, out_bytes, erase_b, nk * es) ||
                                            overlaps(out, out_bytes, write_w, nv * es))) ||
        overlaps(out, out_bytes, state_in, nst * 4) || overlaps(out, out_bytes, state_out, nst * 4))
        return LAM_ERR_INVALID_ARG;
    if (state_out && state_in && state_out != state_in &&
        overlaps(state_out, nst * 4, state_in, nst * 4))
        return LAM_ERR_INVALID_ARG;

    lam::DeltaArgs a = shape_args(variant, dtype, B, T, H, dk, dv);
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = variant == LAM_DELTANET ? nullptr : alpha;
    a.erase_b = variant == LAM_GATED_DELTANET2 ? erase_b : nullptr;
    a.write_w = variant == LAM_GATED_DELTANET2 ? write_w : nullptr;
    a.beta = beta;
    a.state_in = state_in;
    a.out = out;
    a.state_out = state_out;

    Schedule sched;
    size_t need;
    st = plan_delta(a, algo, &sched, &need);
    if (st != LAM_OK) return st;
    a.side = side_out;
    a.side_kind = side;
    const void *args[] = {q, k, v, a.alpha, a.erase_b, a.write_w, beta, state_in, out, state_out, side_out};
    const int64_t arg_bytes[] = {nk * es, nk * es, nv * es, alpha_bytes, nk * es, nv * es, ns * es,
                                 nst * 4, out_bytes, nst * 4, out_bytes};
    if (!workspace_ok(workspace, workspace_bytes, need, args, arg_bytes, 11)) return LAM_ERR_INVALID_ARG;
    a.ws = need ? workspace : nullptr;

    if (T == 0 && !state_out) return LAM_OK;
    if (sched == kChunked) return from_hip(lam::launch_delta_chunked(a, stream));
    return from_hip(lam::launch_delta_recurrent(a, stream));
}

int64_t lam_loglinear_levels(int64_t last_position) {
    if (last_position < 1) return 1;
    int64_t n = 1;
    while (n < 63 && (INT64_C(1) << (n - 1)) <= last_position) ++n;  // floor(log2) + 2
    return n;
}

lam_status lam_loglinear_forward(int variant, int dtype, int64_t B, int64_t T, int64_t H, int64_t dk,
                                 int64_t dv, int64_t nL, int64_t t0, const void *q, const void *k,
                                 const void *v, const void *alpha, const void *erase_b,
                                 const void *write_w, const void *beta, const float *lam,
                                 const float *state_in, void *out, float *state_out,
                                 hipStream_t stream) {
    lam_status st = check_delta_shape(variant, dtype, B, T, H, dk, dv, LAM_ALGO_RECURRENT);
    if (st != LAM_OK) return st;
    if (nL < 1 || t0 < 0) return LAM_ERR_INVALID_ARG;
    if (nL > lam::kLogLinMaxLevels) return LAM_ERR_UNSUPPORTED;
    if (t0 > (INT64_C(1) << (lam::kLogLinMaxLevels - 1)) - 1 - T) return LAM_ERR_UNSUPPORTED;  // positions
    const int64_t last = t0 + T - 1;
    if (T > 0 && nL < lam_loglinear_levels(last)) return LAM_ERR_INVALID_ARG;  // too few levels
    lam::DeltaArgs a = shape_args(variant, dtype, B, T, H, dk, dv);
    if (!lam::loglin_supported(a, static_cast<int>(nL))) return LAM_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return LAM_OK;
    int64_t nk, nv, ns, nst, nlv, nlam;
    elems(B, T, H, dk, nk);
    elems(B, T, H, dv, nv);
    elems(B, T, H, 1, ns);
    elems(B, 1, H, dk * dv, nst);
    if (!mul_ok(nst, nL, nlv) || !mul_ok(ns, nL, nlam)) return LAM_ERR_INVALID_ARG;
    if (T > 0) {
        if (!q || !k || !v || !beta || !lam || !out) return LAM_ERR_INVALID_ARG;
        if (variant != LAM_DELTANET && !alpha) return LAM_ERR_INVALID_ARG;
        if (variant == LAM_GATED_DELTANET2 && (!erase_b || !write_w)) return LAM_ERR_INVALID_ARG;
    }
    const int64_t es = dtype == LAM_BF16 ? 2 : 4;
    const bool gated = variant != LAM_DELTANET, g2 = variant == LAM_GATED_DELTANET2;
    const void *ins[] = {q, k, v, gated ? alpha : nullptr, g2 ? erase_b : nullptr, g2 ? write_w : nullptr,
                         beta, lam, state_in};
    const int64_t inb[] = {nk * es, nk * es, nv * es, (variant == LAM_KIMI_DELTA ? nk : ns) * es, nk * es,
                           nv * es, ns * es, nlam * 4, nlv * 4};
    for (int i = 0; i < 9; ++i) {
        if (overlaps(out, nv * es, ins[i], inb[i])) return LAM_ERR_INVALID_ARG;
        if (i < 8 && overlaps(state_out, nlv * 4, ins[i], inb[i])) return LAM_ERR_INVALID_ARG;
    }
    if (overlaps(out, nv * es, state_out, nlv * 4)) return LAM_ERR_INVALID_ARG;
    if (state_out && state_in && state_out != state_in && overlaps(state_out, nlv * 4, state_in, nlv * 4))
        return LAM_ERR_INVALID_ARG;
    if (T == 0 && !state_out) return LAM_OK;
    lam::LogLinArgs g{};
    g.f = a;
    g.f.q = q;
    g.f.k = k;
    g.f.v = v;
    g.f.alpha = gated ? alpha : nullptr;
    g.f.erase_b = g2 ? erase_b : nullptr;
    g.f.write_w = g2 ? write_w : nullptr;
    g.f.beta = beta;
    g.f.state_in = state_in;
    g.f.out = out;
    g.f.state_out = state_out;
    g.nL = static_cast<int>(nL);
    g.t0 = t0;
    g.lam = lam;
    return from_hip(lam::launch_loglin(g, stream));
}

lam_status lam_loglinear_lambda(int dtype, int64_t M, int64_t nL, int64_t nh, const void *d,
                                const float *W1, const float *W2, const float *b, float *lam,
                                hipStream_t stream) {
    if (dtype != LAM_F32 && dtype != LAM_BF16) return LAM_ERR_INVALID_ARG;
    if (M < 0 || nL < 1 || nh < 1) return LAM_ERR_INVALID_ARG;
    if (nL > lam::kLogLinMaxLevels || nh > lam::kLogLinMaxHidden) return LAM_ERR_UNSUPPORTED;
    int64_t n;
    if (!mul_ok(M, nL, n) || (M + 255) / 256 > INT_MAX) return LAM_ERR_INVALID_ARG;
    if (M == 0) return LAM_OK;
    if (!d || !W1 || !W2 || !b || !lam) return LAM_ERR_INVALID_ARG;
    const int64_t es = dtype == LAM_BF16 ? 2 : 4;
    if (overlaps(lam, n * 4, d, n * es) || overlaps(lam, n * 4, W1, nL * nh * 4) ||
        overlaps(lam, n * 4, W2, nL * nh * 4) || overlaps(lam, n * 4, b, nL * 4))
        return LAM_ERR_INVALID_ARG;
    return from_hip(lam::launch_loglin_lambda(dtype, M, static_cast<int>(nL), static_cast<int>(nh), d, W1, W2,
                                              b, lam, stream));
}

lam_status lam_route(int dtype, int64_t M, int64_t D, int64_t N, const void *s, const void *P, void *h,
                     hipStream_t stream) {
    if (dtype != LAM_F32 && dtype != LAM_BF16) return LAM_ERR_INVALID_ARG;
    if (M < 0 || D <= 0 || N <= 0) return LAM_ERR_INVALID_ARG;
    if (!lam::route_supported(D, N)) return LAM_ERR_UNSUPPORTED;
    int64_t ns, nh, np;
    // sizes, 32-bit column indices and the grid (128 x 128 tiles)
    if (!mul_ok(M, N, ns) || !mul_ok(M, D, nh) || !mul_ok(D, N, np)) return LAM_ERR_INVALID_ARG;
    if (D > INT_MAX / 2 || N > INT_MAX / 2) return LAM_ERR_INVALID_ARG;
    if (((M + 127) / 128) * ((D + 127) / 128) > INT_MAX) return LAM_ERR_INVALID_ARG;
    if (M == 0) return LAM_OK;
    if (!s || !P || !h) return LAM_ERR_INVALID_ARG;
    // rows are read as 16-byte pieces
    const auto al = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    if (!al(s) || !al(P) || !al(h)) return LAM_ERR_INVALID_ARG;
    const int64_t es = dtype == LAM_BF16 ? 2 : 4;
    if (overlaps(h, nh * es, s, ns * es) || overlaps(h, nh * es, P, np * es)) return LAM_ERR_INVALID_ARG;
    return from_hip(lam::launch_route(dtype, M, D, N, s, P, h, stream));
}

namespace {
// The backward schedule of a validated call: chunked (fp32 matrix cores) or
// token-recurrent, and its workspace.
lam_status plan_backward(const lam::DeltaArgs &a, int algo, bool *chunked, size_t *bytes) {
    *chunked = false;
    *bytes = 0;
    if (a.B == 0 || a.H == 0) return LAM_OK;
    const bool chunked_ok = lam::delta_f32_chunked_supported(a);
    if (algo == LAM_ALGO_CHUNKED && !chunked_ok) return LAM_ERR_UNSUPPORTED;
    *chunked = chunked_ok && a.T > 0 && algo != LAM_ALGO_RECURRENT;
    const bool ok = *chunked ? lam::delta_f32_backward_workspace(a, bytes) : lam::delta_backward_workspace(a, bytes);
    return ok ? LAM_OK : LAM_ERR_UNSUPPORTED;
}
}  // namespace

lam_status lam_backward_workspace_size(int variant, int dtype, int64_t B, int64_t T, int64_t H,
                                       int64_t dk, int64_t dv, int algo, size_t *bytes) {
    if (!bytes) return LAM_ERR_INVALID_ARG;
    *bytes = 0;
    lam_status st = check_delta_shape(variant, dtype, B, T, H, dk, dv, algo);
    if (st != LAM_OK) return st;
    bool chunked;
    return plan_backward(shape_args(variant, dtype, B, T, H, dk, dv), algo, &chunked, bytes);
}

lam_status lam_backward(int variant, int dtype, int64_t B, int64_t T, int64_t H, int64_t dk,
                        int64_t dv, const void *q, const void *k, const void *v,
                        const void *alpha, const void *erase_b, const void *write_w,
                        const void *beta, const float *state_in, const void *dout,
                        const float *dstate_out, float *dq, float *dk_, float *dv_, float *dalpha,
                        float *derase_b, float *dwrite_w, float *dbeta, float *dstate_in, int algo,
                        void *workspace, size_t workspace_bytes, hipStream_t stream) {
    size_t need = 0;
    lam_status st = lam_backward_workspace_size(variant, dtype, B, T, H, dk, dv, algo, &need);
    if (st != LAM_OK) return st;
    if (B == 0 || H == 0) return LAM_OK;
    bool chunked;
    plan_backward(shape_args(variant, dtype, B, T, H, dk, dv), algo, &chunked, &need);
    int64_t nk, nv, ns, nst;
    elems(B, T, H, dk, nk);
    elems(B, T, H, dv, nv);
    elems(B, T, H, 1, ns);
    elems(B, 1, H, dk * dv, nst);
    const bool gated = variant != LAM_DELTANET, g2 = variant == LAM_GATED_DELTANET2;
    if (T > 0) {
        if (!q || !k || !v || !beta || !dout || !dq || !dk_ || !dv_ || !dbeta) return LAM_ERR_INVALID_ARG;
        if (gated && (!alpha || !dalpha)) return LAM_ERR_INVALID_ARG;
        if (g2 && (!erase_b || !write_w || !derase_b || !dwrite_w)) return LAM_ERR_INVALID_ARG;
    }
    const int64_t es = dtype == LAM_BF16 ? 2 : 4;
    const int64_t na = variant == LAM_KIMI_DELTA ? nk : ns;
    const void *ins[] = {q, k, v, gated ? alpha : nullptr, g2 ? erase_b : nullptr, g2 ? write_w : nullptr,
                         beta, state_in, dout, dstate_out};
    const int64_t inb[] = {nk * es, nk * es, nv * es, na * es, nk * es, nv * es, ns * es, nst * 4, nv * es, nst * 4};
    void *outs[] = {dq, dk_, dv_, gated ? dalpha : nullptr, g2 ? derase_b : nullptr, g2 ? dwrite_w : nullptr,
                    dbeta, dstate_in};
    const int64_t outb[] = {nk * 4, nk * 4, nv * 4, na * 4, nk * 4, nv * 4, ns * 4, nst * 4};
    for (int o = 0; o < 8; ++o) {
        for (int i = 0; i < 10; ++i)
            if (overlaps(outs[o], outb[o], ins[i], inb[i])) return LAM_ERR_INVALID_ARG;
        for (int o2 = o + 1; o2 < 8; ++o2)
            if (overlaps(outs[o], outb[o], outs[o2], outb[o2])) return LAM_ERR_INVALID_ARG;
    }
    const void *all[18];
    int64_t allb[18];
    for (int i = 0; i < 10; ++i) all[i] = ins[i], allb[i] = inb[i];
    for (int o = 0; o < 8; ++o) all[10 + o] = outs[o], allb[10 + o] = outb[o];
    if (!workspace_ok(workspace, workspace_bytes, need, all, allb, 18)) return LAM_ERR_INVALID_ARG;
    if (T == 0 && !dstate_in) return LAM_OK;  // (T = 0: dstate_in = dstate_out, or zero)
    lam::DeltaBwdArgs g{};
    g.f = shape_args(variant, dtype, B, T, H, dk, dv);
    g.f.q = q;
    g.f.k = k;
    g.f.v = v;
    g.f.alpha = gated ? alpha : nullptr;
    g.f.erase_b = g2 ? erase_b : nullptr;
    g.f.write_w = g2 ? write_w : nullptr;
    g.f.beta = beta;
    g.f.state_in = state_in;
    g.f.ws = workspace;
    g.dout = dout;
    g.dstate_out = dstate_out;
    g.dq = dq;
    g.dk = dk_;
    g.dv = dv_;
    g.dalpha = gated ? dalpha : nullptr;
    g.derase_b = g2 ? derase_b : nullptr;
    g.dwrite_w = g2 ? dwrite_w : nullptr;
    g.dbeta = dbeta;
    g.dstate_in = dstate_in;
    g.ckpt = reinterpret_cast<float *>(static_cast<char *>(workspace) + lam::kStatusBytes);
    if (chunked) return from_hip(lam::launch_delta_f32_backward(g, stream));
    return from_hip(lam::launch_delta_backward(g, stream));
}

lam_status lam_step(int variant, int dtype, int64_t N, int64_t H, int64_t dk, int64_t dv,
                    const void *q, const void *k, const void *v, const void *alpha,
                    const void *erase_b, const void *write_w, const void *beta, float *state,
                    void *out, hipStream_t stream) {
    lam_status st = check_delta_shape(variant, dtype, N, 1, H, dk, dv, LAM_ALGO_RECURRENT);
    if (st != LAM_OK) return st;
    if (N == 0 || H == 0) return LAM_OK;
    if (!state) return LAM_ERR_INVALID_ARG;
    lam::DeltaArgs a = shape_args(variant, dtype, N, 1, H, dk, dv);
    if (!lam::delta_step_supported(a))  // dk = 96: the token-recurrent kernel, one token
        return lam_forward(variant, dtype, N, 1, H, dk, dv, q, k, v, alpha, erase_b, write_w, beta,
                           state, out, state, nullptr, 0, LAM_ALGO_RECURRENT, stream);
    // the argument checks of a one-token lam_forward (no workspace: recurrent)
    int64_t nk, nv, ns, nst;
    elems(N, 1, H, dk, nk);
    elems(N, 1, H, dv, nv);
    elems(N, 1, H, 1, ns);
    elems(N, 1, H, dk * dv, nst);
    if (!q || !k || !v || !beta || !out) return LAM_ERR_INVALID_ARG;
    if (variant != LAM_DELTANET && !alpha) return LAM_ERR_INVALID_ARG;
    if (variant == LAM_GATED_DELTANET2 && (!erase_b || !write_w)) return LAM_ERR_INVALID_ARG;
    const int64_t es = dtype == LAM_BF16 ? 2 : 4;
    const int64_t ob = nv * es;
    const int64_t alpha_bytes = (variant == LAM_KIMI_DELTA ? nk : ns) * es;
    if (overlaps(out, ob, q, nk * es) || overlaps(out, ob, k, nk * es) || overlaps(out, ob, v, nv * es) ||
        overlaps(out, ob, beta, ns * es) ||
        (variant != LAM_DELTANET && overlaps(out, ob, alpha, alpha_bytes)) ||
        (variant == LAM_GATED_DELTANET2 &&
         (overlaps(out, ob, erase_b, nk * es) || overlaps(out, ob, write_w, nv * es))) ||
        overlaps(out, ob, state, nst * 4))
        return LAM_ERR_INVALID_ARG;
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = variant == LAM_DELTANET ? nullptr : alpha;
    a.erase_b = variant == LAM_GATED_DELTANET2 ? erase_b : nullptr;
    a.write_w = variant == LAM_GATED_DELTANET2 ? write_w : nullptr;
    a.beta = beta;
    a.state_in = state;
    a.out = out;
    a.state_out = state;
    return from_hip(lam::launch_delta_step(a, stream));
}

lam_status lam_vla_step(int dtype, int64_t N, int64_t H, int64_t d, const void *q, const void *k,
                        const void *v, const void *p, float *A, float *S, void *out,
                        hipStream_t stream) {
    lam_status st = check_vla_shape(dtype, N, 1, H, d, LAM_ALGO_RECURRENT);
    if (st != LAM_OK) return st;
    if (N == 0 || H == 0) return LAM_OK;
    if (!A || !S) return LAM_ERR_INVALID_ARG;
    return lam_vla_forward(dtype, N, 1, H, d, q, k, v, p, A, S, out, A, S, nullptr, 0,
                           LAM_ALGO_RECURRENT, stream);
}

lam_status lam_vla_forward_ratio(int dtype, int64_t B, int64_t T, int64_t H, int64_t d, const void *q,
                                 const void *k, const void *v, const void *p, const float *A_in,
                                 const float *S_in, const float *n_in, void *out, float *A_out, float *S_out,
                                 float *n_out, hipStream_t stream) {
    lam_status st = check_vla_shape(dtype, B, T, H, d, LAM_ALGO_RECURRENT);
    if (st != LAM_OK) return st;
    if (B == 0 || H == 0) return LAM_OK;
    int64_t n, nst;
    elems(B, T, H, d, n);
    elems(B, 1, H, d * d, nst);
    const int64_t nnb = B * H * d * 4;  // bytes of n
    if (T > 0 && (!q || !k || !v || !p || !out)) return LAM_ERR_INVALID_ARG;
    const int64_t es = dtype == LAM_BF16 ? 2 : 4;
    const int64_t ob = n * es;
    const void *all[] = {q, k, v, p, A_in, S_in, n_in, A_out, S_out, n_out};
    const int64_t all_b[] = {ob, ob, ob, ob, nst * 4, nst * 4, nnb, nst * 4, nst * 4, nnb};
    for (int i = 0; i < 10; ++i)
        if (overlaps(out, ob, all[i], all_b[i])) return LAM_ERR_INVALID_ARG;
    const float *ins[3] = {A_in, S_in, n_in};
    const int64_t in_b[3] = {nst * 4, nst * 4, nnb};
    float *outs[3] = {A_out, S_out, n_out};
    const int64_t out_b[3] = {nst * 4, nst * 4, nnb};
    for (int o = 0; o < 3; ++o) {
        for (int i = 0; i < 3; ++i)  // an output may be its own input's buffer, nothing else
            if (outs[o] && ins[i] && !(o == i && outs[o] == ins[i]) && overlaps(outs[o], out_b[o], ins[i], in_b[i]))
                return LAM_ERR_INVALID_ARG;
        for (int o2 = o + 1; o2 < 3; ++o2)
            if (outs[o] && outs[o2] && overlaps(outs[o], out_b[o], outs[o2], out_b[o2])) return LAM_ERR_INVALID_ARG;
    }
    if (T == 0 && !A_out && !S_out && !n_out) return LAM_OK;
    lam::VlaArgs a{};
    a.dtype = dtype;
    a.B = B;
    a.T = T;
    a.H = H;
    a.d = static_cast<int>(d);
    a.q = q;
    a.k = k;
    a.v = v;
    a.p = p;
    a.A_in = A_in;
    a.S_in = S_in;
    a.out = out;
    a.A_out = A_out;
    a.S_out = S_out;
    a.ratio = true;
    a.n_in = n_in;
    a.n_out = n_out;
    return from_hip(lam::launch_vla_recurrent(a, stream));
}

lam_status lam_vla_step_ratio(int dtype, int64_t N, int64_t H, int64_t d, const void *q, const void *k,
                              const void *v, const void *p, float *A, float *S, float *n, void *out,
                              hipStream_t stream) {
    lam_status st = check_vla_shape(dtype, N, 1, H, d, LAM_ALGO_RECURRENT);
    if (st != LAM_OK) return st;
    if (N == 0 || H == 0) return LAM_OK;
    if (!A || !S || !n) return LAM_ERR_INVALID_ARG;
    return lam_vla_forward_ratio(dtype, N, 1, H, d, q, k, v, p, A, S, n, out, A, S, n, stream);
}

lam_status lam_vla_workspace_size(int dtype, int64_t B, int64_t T, int64_t H, int64_t d, int algo,
                                  size_t *bytes) {
    if (!bytes) return LAM_ERR_INVALID_ARG;
    *bytes = 0;
    lam_status st = check_vla_shape(dtype, B, T, H, d, algo);
    if (st != LAM_OK) return st;
    lam::VlaArgs a{};
    a.dtype = dtype;
    a.B = B;
    a.T = T;
    a.H = H;
    a.d = static_cast<int>(d);
    Schedule sched;
    return plan_vla(a, algo, &sched, bytes);
}

lam_status lam_vla_forward(int dtype, int64_t B, int64_t T, int64_t H, int64_t d,
                           const void *q, const void *k, const void *v, const void *p,
                           const float *A_in, const float *S_in, void *out, float *A_out,
                           float *S_out, void *workspace, size_t workspace_bytes, int algo,
                           hipStream_t stream) {
    lam_status st = check_vla_shape(dtype, B, T, H, d, algo);
    if (st != LAM_OK) return st;
    if (B == 0 || H == 0) return LAM_OK;
    int64_t n, nst;
    elems(B, T, H, d, n);
    elems(B, 1, H, d * d, nst);
    if (T > 0 && (!q || !k || !v || !p || !out)) return LAM_ERR_INVALID_ARG;
    const int64_t es = dtype == LAM_BF16 ? 2 : 4;
    const int64_t ob = n * es;
    if (overlaps(out, ob, q, ob) || overlaps(out, ob, k, ob) || overlaps(out, ob, v, ob) ||
        overlaps(out, ob, p, ob) || overlaps(out, ob, A_in, nst * 4) ||
        overlaps(out, ob, S_in, nst * 4) || overlaps(out, ob, A_out, nst * 4) ||
        overlaps(out, ob, S_out, nst * 4))
        return LAM_ERR_INVALID_ARG;
    const float *ins[2] = {A_in, S_in};
    float *outs[2] = {A_out, S_out};
    for (float *o : outs)
        for (const float *i : ins)
            if (o && i && o != i && overlaps(o, nst * 4, i, nst * 4)) return LAM_ERR_INVALID_ARG;
    if (A_out && S_out && overlaps(A_out, nst * 4, S_out, nst * 4)) return LAM_ERR_INVALID_ARG;

    lam::VlaArgs a{};
    a.dtype = dtype;
    a.B = B;
    a.T = T;
    a.H = H;
    a.d = static_cast<int>(d);
    a.q = q;
    a.k = k;
    a.v = v;
    a.p = p;
    a.A_in = A_in;
    a.S_in = S_in;
    a.out = out;
    a.A_out = A_out;
    a.S_out = S_out;
    Schedule sched;
    size_t need;
    st = plan_vla(a, algo, &sched, &need);
    if (st != LAM_OK) return st;
    const void *args[] = {q, k, v, p, A_in, S_in, out, A_out, S_out};
    const int64_t arg_bytes[] = {ob, ob, ob, ob, nst * 4, nst * 4, ob, nst * 4, nst * 4};
    if (!workspace_ok(workspace, workspace_bytes, need, args, arg_bytes, 9)) return LAM_ERR_INVALID_ARG;
    a.ws = need ? workspace : nullptr;
    if (T == 0 && !A_out && !S_out) return LAM_OK;
    if (sched == kChunked) return from_hip(lam::launch_vla_chunked(a, stream));
    return from_hip(lam::launch_vla_recurrent(a, stream));
}

}  // extern "C"
