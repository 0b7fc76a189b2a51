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

}  // namespace

extern "C" {

const char *lam_status_string(lam_status s) {
    switch (s) {
        case LAM_OK: return "ok";
        case LAM_ERR_INVALID_ARG: return "invalid argument";
        case LAM_ERR_UNSUPPORTED: return "unsupported shape, dtype or algorithm";
        case LAM_ERR_HIP: return "HIP launch failure";
    }
    return "unknown status";
}

int lam_abi_version(void) { return 100; }

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

lam_status lam_forward(int variant, int dtype, int64_t B, int64_t T, int64_t H, int64_t dk,
                       int64_t dv, const void *q, const void *k, const void *v,
                       const void *alpha, const void *erase_b, const void *write_w,
                       const void *beta, const float *state_in, void *out, float *state_out,
                       int algo, hipStream_t stream) {
    if (variant < LAM_DELTANET || variant > LAM_GATED_DELTANET2) return LAM_ERR_INVALID_ARG;
    if (dtype != LAM_F32 && dtype != LAM_BF16) return LAM_ERR_INVALID_ARG;
    if (algo < LAM_ALGO_AUTO || algo > LAM_ALGO_CHUNKED) return LAM_ERR_INVALID_ARG;
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return LAM_ERR_INVALID_ARG;
    if (!supported_head(dk) || !supported_head(dv)) return LAM_ERR_UNSUPPORTED;
    int64_t nk, nv, ns, nst;
    if (!elems(B, T, H, dk, nk) || !elems(B, T, H, dv, nv) || !elems(B, T, H, 1, ns) ||
        !elems(B, 1, H, dk * dv, nst))
        return LAM_ERR_INVALID_ARG;
    // grid and 32-bit in-chain indices
    if (B * H > (INT64_C(1) << 24) || T > INT_MAX / 2) return LAM_ERR_INVALID_ARG;
    if (B == 0 || H == 0) return LAM_OK;
    const bool need_state_copy = T == 0;
    if (!need_state_copy) {
        if (!q || !k || !v || !beta || !out) return LAM_ERR_INVALID_ARG;
        if (variant != LAM_DELTANET && !alpha) return LAM_ERR_INVALID_ARG;
        if (variant == LAM_GATED_DELTANET2 && (!erase_b || !write_w)) return LAM_ERR_INVALID_ARG;
    }
    const int64_t es = dtype == LAM_BF16 ? 2 : 4;
    const int64_t out_bytes = nv * es;
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

    lam::DeltaArgs a;
    a.variant = variant;
    a.dtype = dtype;
    a.B = B;
    a.T = T;
    a.H = H;
    a.dk = static_cast<int>(dk);
    a.dv = static_cast<int>(dv);
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

    if (T == 0 && !state_out) return LAM_OK;
    if (algo == LAM_ALGO_CHUNKED) {
        if (!lam::delta_chunked_supported(a)) return LAM_ERR_UNSUPPORTED;
        return from_hip(lam::launch_delta_chunked(a, stream));
    }
    if (algo == LAM_ALGO_AUTO && T > 0 && lam::delta_chunked_supported(a))
        return from_hip(lam::launch_delta_chunked(a, stream));
    return from_hip(lam::launch_delta_recurrent(a, stream));
}

lam_status lam_vla_forward(int dtype, int64_t B, int64_t T, int64_t H, int64_t d,
                           const void *q, const void *k, const void *v, const void *p,
                           const float *A_in, const float *S_in, void *out, float *A_out,
                           float *S_out, int algo, hipStream_t stream) {
    if (dtype != LAM_F32 && dtype != LAM_BF16) return LAM_ERR_INVALID_ARG;
    if (algo < LAM_ALGO_AUTO || algo > LAM_ALGO_CHUNKED) return LAM_ERR_INVALID_ARG;
    if (B < 0 || T < 0 || H < 0 || d <= 0) return LAM_ERR_INVALID_ARG;
    if (!supported_head(d)) return LAM_ERR_UNSUPPORTED;
    int64_t n, nst;
    if (!elems(B, T, H, d, n) || !elems(B, 1, H, d * d, nst)) return LAM_ERR_INVALID_ARG;
    if (B * H > (INT64_C(1) << 24) || T > INT_MAX / 2) return LAM_ERR_INVALID_ARG;
    if (B == 0 || H == 0) return LAM_OK;
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

    lam::VlaArgs a;
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
    if (T == 0 && !A_out && !S_out) return LAM_OK;
    if (algo != LAM_ALGO_RECURRENT && T > 0 && lam::vla_chunked_supported(a))
        return from_hip(lam::launch_vla_chunked(a, stream));
    if (algo == LAM_ALGO_CHUNKED && T > 0) return LAM_ERR_UNSUPPORTED;
    return from_hip(lam::launch_vla_recurrent(a, stream));
}

}  // extern "C"
