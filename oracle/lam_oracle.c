/*
 * lam_oracle.c -- plain, slow, token-by-token CPU oracle for the causal
 * recurrent-memory linear-attention forward scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library; the two meet only through seeded inputs.
 *
 * Sources (cited by page title and section; the pages are web articles):
 *   [LA-arch]  "Mechanisms, trade-offs and cross-layer routing of
 *              linear-attention architectures" (aitrends.kr), sections
 *              "Key contributions", "Understanding the core idea",
 *              "Methodology" and "Technical details": the unified
 *              recurrent-memory notation (memory W in R^{dv x dk}, read
 *              y = W phi(q)), the DeltaNet delta rule, Gated DeltaNet's
 *              scalar decay, Kimi Delta's channel-wise decay on the
 *              key-feature axis and Gated DeltaNet-2's channel-wise erase
 *              and write gates.
 *   [VLA]      "Technical summary: Variational Linear Attention (VLA)"
 *              (gist.science), section 2.2 (inverse penalty A = M^{-1} kept
 *              by Sherman-Morrison at O(d^2) per step), section 2.3 (the
 *              three recursive update rules; unit-length k-hat and alpha-hat;
 *              ELU+1 feature map).
 *
 * Every quantity is computed in `real` (double unless the file is compiled
 * with -DLAM_ORACLE_REAL=float, which gives the single-precision spread
 * check).  Inputs and outputs are always double arrays; a float build rounds
 * each input once on load.
 *
 * Readings taken where the pages are silent:
 *   - the read happens after the update: y_t = W_t q_t (and S_t q-hat_t);
 *   - Gated DeltaNet's residual is taken against the decayed memory,
 *     r = v - (alpha W_{t-1}) k;
 *   - Kimi Delta's decay multiplies the key-channel columns: W diag(alpha_t);
 *   - Gated DeltaNet-2 reads with the erase direction e = b*k against the
 *     decayed memory, targets z = w*v and writes along k;
 *   - VLA's Sherman-Morrison vector u_t is the penalty direction p_t, with
 *     z_t = A_{t-1} p_t; the output is S_t q-hat_t with no denominator;
 *   - no 1/sqrt(d) scale and no epsilon in any norm.
 *
 * Parity status: every function here is pinned by closed forms, special
 * cases, invariants and brute force in the CPU test tier; no function is
 * unpinned.
 */
#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

#ifndef LAM_ORACLE_REAL
#define LAM_ORACLE_REAL double
#endif
typedef LAM_ORACLE_REAL real;

/* Variant codes of the oracle's own interface. */
enum {
    ORACLE_DELTANET = 0,      /* alpha = 1                                  */
    ORACLE_GATED_DELTANET = 1, /* scalar alpha per (b, t, h)                */
    ORACLE_KIMI_DELTA = 2,    /* alpha per (b, t, h, key channel)          */
    ORACLE_GATED_DELTANET2 = 3 /* scalar alpha + erase b[dk], write w[dv]   */
};

/* Per-token side output of the delta-rule forward ([LA-arch] "Methodology"
   and "Technical details", cross-layer routing): the internal signal s that
   CLER / CLER-H route is the delta-rule residual r, the one CLVR routes is
   the write value (v, or the write target z = w*v for Gated DeltaNet-2). */
enum { ORACLE_SIDE_NONE = 0, ORACLE_SIDE_RESIDUAL = 1, ORACLE_SIDE_VALUE = 2 };

/* Row-major index helpers for [B,T,H,n] token streams and [B,H,r,c] states. */
static size_t tok(long b, long t, long h, long T, long H, long n) {
    return (((size_t)b * T + t) * H + h) * (size_t)n;
}
static size_t st(long b, long h, long H, long r, long c) {
    return ((size_t)b * H + h) * (size_t)r * (size_t)c;
}

/*
 * Delta-rule family, one (b, h) chain.  Per token, in this order
 * ([LA-arch] Technical details / Methodology):
 *   decay     W~ = alpha W            (Gated DeltaNet, Gated DeltaNet-2)
 *             W~ = W diag(alpha)      (Kimi Delta: key-feature channels)
 *             W~ = W                  (DeltaNet)
 *   predict   vbar = W~ kk,  kk = k   (kk = b*k for Gated DeltaNet-2)
 *   residual  r = target - vbar,  target = v  (z = w*v for Gated DeltaNet-2)
 *   write     W = W~ + beta r k^T
 *   read      y = W q
 * With drop_delta set the prediction is skipped (r = target): that is the
 * plain additive accumulation the VLA page contrasts against (section 2.1),
 * used only as a test hook.
 */
static void delta_chain(int variant, long b, long h, long T, long H, long dk,
                        long dv, const double *q, const double *k,
                        const double *v, const double *alpha,
                        const double *erase_b, const double *write_w,
                        const double *beta, const double *state_in,
                        double *out, double *state_out, int drop_delta,
                        double *side, int side_kind,
                        real *W, real *kk, real *target, real *r) {
    for (long i = 0; i < dv * dk; ++i)
        W[i] = state_in ? (real)state_in[st(b, h, H, dv, dk) + i] : (real)0;

    for (long t = 0; t < T; ++t) {
        const double *kt = k + tok(b, t, h, T, H, dk);
        const double *qt = q + tok(b, t, h, T, H, dk);
        const double *vt = v + tok(b, t, h, T, H, dv);
        const real bt = (real)beta[tok(b, t, h, T, H, 1)];

        /* decay */
        if (variant == ORACLE_GATED_DELTANET || variant == ORACLE_GATED_DELTANET2) {
            const real a = (real)alpha[tok(b, t, h, T, H, 1)];
            for (long i = 0; i < dv * dk; ++i) W[i] = a * W[i];
        } else if (variant == ORACLE_KIMI_DELTA) {
            const double *at = alpha + tok(b, t, h, T, H, dk);
            for (long i = 0; i < dv; ++i)
                for (long j = 0; j < dk; ++j) W[i * dk + j] = W[i * dk + j] * (real)at[j];
        }

        /* read key and write target */
        for (long j = 0; j < dk; ++j) kk[j] = (real)kt[j];
        for (long i = 0; i < dv; ++i) target[i] = (real)vt[i];
        if (variant == ORACLE_GATED_DELTANET2) {
            const double *bt_ = erase_b + tok(b, t, h, T, H, dk);
            const double *wt_ = write_w + tok(b, t, h, T, H, dv);
            for (long j = 0; j < dk; ++j) kk[j] = (real)bt_[j] * kk[j];
            for (long i = 0; i < dv; ++i) target[i] = (real)wt_[i] * target[i];
        }

        /* residual against the (decayed) memory */
        for (long i = 0; i < dv; ++i) {
            real pred = 0;
            if (!drop_delta)
                for (long j = 0; j < dk; ++j) pred += W[i * dk + j] * kk[j];
            r[i] = target[i] - pred;
        }

        /* cross-layer routing signal of this token: the residual (CLER) or
           the write value (CLVR) */
        if (side) {
            double *sd = side + tok(b, t, h, T, H, dv);
            for (long i = 0; i < dv; ++i)
                sd[i] = (double)(side_kind == ORACLE_SIDE_RESIDUAL ? r[i] : target[i]);
        }

        /* write along the key */
        for (long i = 0; i < dv; ++i)
            for (long j = 0; j < dk; ++j) W[i * dk + j] += bt * r[i] * (real)kt[j];

        /* read with the query */
        double *yt = out + tok(b, t, h, T, H, dv);
        for (long i = 0; i < dv; ++i) {
            real acc = 0;
            for (long j = 0; j < dk; ++j) acc += W[i * dk + j] * (real)qt[j];
            yt[i] = (double)acc;
        }
    }
    if (state_out)
        for (long i = 0; i < dv * dk; ++i) state_out[st(b, h, H, dv, dk) + i] = (double)W[i];
}

/*
 * oracle_delta_forward: the four delta-rule variants over a [B,T] block.
 * Layouts: q, k, erase_b [B,T,H,dk]; v, write_w, out [B,T,H,dv];
 * alpha [B,T,H] (Gated DeltaNet, Gated DeltaNet-2) or [B,T,H,dk] (Kimi
 * Delta) or NULL (DeltaNet); beta [B,T,H]; state_in / state_out
 * [B,H,dv,dk] (NULL in = zero memory, NULL out = not written).
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_delta_forward_side(int variant, long B, long T, long H, long dk, long dv,
                              const double *q, const double *k, const double *v,
                              const double *alpha, const double *erase_b,
                              const double *write_w, const double *beta,
                              const double *state_in, double *out,
                              double *state_out, int drop_delta, double *side,
                              int side_kind, int nthreads);

int oracle_delta_forward(int variant, long B, long T, long H, long dk, long dv,
                         const double *q, const double *k, const double *v,
                         const double *alpha, const double *erase_b,
                         const double *write_w, const double *beta,
                         const double *state_in, double *out,
                         double *state_out, int drop_delta, int nthreads) {
    return oracle_delta_forward_side(variant, B, T, H, dk, dv, q, k, v, alpha, erase_b, write_w,
                                     beta, state_in, out, state_out, drop_delta, NULL,
                                     ORACLE_SIDE_NONE, nthreads);
}

/*
 * oracle_delta_forward_side: oracle_delta_forward that also writes the
 * per-token routing signal to side [B,T,H,dv] (side_kind RESIDUAL: r;
 * VALUE: the write value; NONE with side NULL: nothing).
 */
int oracle_delta_forward_side(int variant, long B, long T, long H, long dk, long dv,
                              const double *q, const double *k, const double *v,
                              const double *alpha, const double *erase_b,
                              const double *write_w, const double *beta,
                              const double *state_in, double *out,
                              double *state_out, int drop_delta, double *side,
                              int side_kind, int nthreads) {
    if (side_kind < ORACLE_SIDE_NONE || side_kind > ORACLE_SIDE_VALUE) return -1;
    if ((side_kind == ORACLE_SIDE_NONE) != (side == NULL)) return -1;
    if (variant < ORACLE_DELTANET || variant > ORACLE_GATED_DELTANET2) return -1;
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    if (!q || !k || !v || !beta || !out) return -1;
    if (variant != ORACLE_DELTANET && !alpha) return -1;
    if (variant == ORACLE_GATED_DELTANET2 && (!erase_b || !write_w)) return -1;
    const long chains = B * H;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : omp_get_max_threads()) \
    reduction(| : failed)
    for (long c = 0; c < chains; ++c) {
        real *buf = (real *)malloc(sizeof(real) * (size_t)(dv * dk + 2 * dk + 2 * dv));
        if (!buf) { failed = 1; continue; }
        delta_chain(variant, c / H, c % H, T, H, dk, dv, q, k, v, alpha, erase_b,
                    write_w, beta, state_in, out, state_out, drop_delta, side, side_kind,
                    buf, buf + dv * dk, buf + dv * dk + dk, buf + dv * dk + dk + dv);
        free(buf);
    }
    return failed ? -1 : 0;
}

/*
 * Backward pass of the delta-rule family, one (b, h) chain: the gradients of
 * L = sum_t <dout_t, y_t> + <dstate_out, W_T> with respect to every input,
 * by reverse-mode differentiation of the per-token steps above (the pages
 * give the forward rule only; this is that rule's adjoint, derived here and
 * pinned against central finite differences of oracle_delta_forward).
 *
 * Forward, per token (kk = read key, z = target, W~ = decayed memory):
 *   W~ = decay(W_{t-1});  r = z - W~ kk;  W_t = W~ + beta r k^T;  y_t = W_t q.
 * Reverse, with G the adjoint of W_t (G = dstate_out, or 0, before the last
 * token), for t = T-1 .. 0:
 *   G     += dout_t q^T                         (the read)
 *   dq_t   = W_t^T dout_t
 *   g      = G k                                (rows of G along the write key)
 *   dbeta_t = r . g;  dz = beta g               (the write's scale and target)
 *   dk_t   = beta G^T r + (read key's part of -beta W~^T g)
 *   dW~    = G - beta g kk^T
 *   decay: Gated DeltaNet(-2): dalpha_t = <dW~, W_{t-1}>, G = alpha dW~;
 *          Kimi Delta: dalpha_t[j] = sum_i dW~_ij W_{t-1,ij}, G = dW~ diag(alpha);
 *          DeltaNet: G = dW~.
 *   Gated DeltaNet-2 (kk = b*k, z = w*v): dv = w*dz, dw = v*dz,
 *          dkk = -beta W~^T g, db = k*dkk, dk_t += b*dkk; the others: dv = dz,
 *          dk_t += dkk.
 * After token 0, dstate_in = G.  The forward states W_0 .. W_{T-1} are kept
 * (T dv dk reals per chain), which is the plain way to have them in reverse.
 */
static void delta_chain_bwd(int variant, long b, long h, long T, long H, long dk, long dv,
                            const double *q, const double *k, const double *v,
                            const double *alpha, const double *erase_b,
                            const double *write_w, const double *beta,
                            const double *state_in, const double *dout,
                            const double *dstate_out, double *dq, double *dkg,
                            double *dvg, double *dalpha, double *derase_b,
                            double *dwrite_w, double *dbeta, double *dstate_in,
                            real *Ws, real *Wt, real *G, real *kk, real *z, real *r,
                            real *g, real *dkk) {
    const long n = dv * dk;
    /* forward, keeping W_{t-1} for every t */
    for (long i = 0; i < n; ++i) Ws[i] = state_in ? (real)state_in[st(b, h, H, dv, dk) + i] : (real)0;
    for (long t = 0; t < T; ++t) {
        real *Wp = Ws + t * n, *Wn = Ws + (t + 1) * n;
        const double *kt = k + tok(b, t, h, T, H, dk);
        const double *vt = v + tok(b, t, h, T, H, dv);
        const real bt = (real)beta[tok(b, t, h, T, H, 1)];
        for (long i = 0; i < n; ++i) Wn[i] = Wp[i];
        if (variant == ORACLE_GATED_DELTANET || variant == ORACLE_GATED_DELTANET2) {
            const real a = (real)alpha[tok(b, t, h, T, H, 1)];
            for (long i = 0; i < n; ++i) Wn[i] = a * Wn[i];
        } else if (variant == ORACLE_KIMI_DELTA) {
            const double *at = alpha + tok(b, t, h, T, H, dk);
            for (long i = 0; i < dv; ++i)
                for (long j = 0; j < dk; ++j) Wn[i * dk + j] = Wn[i * dk + j] * (real)at[j];
        }
        for (long j = 0; j < dk; ++j) kk[j] = (real)kt[j];
        for (long i = 0; i < dv; ++i) z[i] = (real)vt[i];
        if (variant == ORACLE_GATED_DELTANET2) {
            const double *bt_ = erase_b + tok(b, t, h, T, H, dk);
            const double *wt_ = write_w + tok(b, t, h, T, H, dv);
            for (long j = 0; j < dk; ++j) kk[j] = (real)bt_[j] * kk[j];
            for (long i = 0; i < dv; ++i) z[i] = (real)wt_[i] * z[i];
        }
        for (long i = 0; i < dv; ++i) {
            real pred = 0;
            for (long j = 0; j < dk; ++j) pred += Wn[i * dk + j] * kk[j];
            r[i] = z[i] - pred;
        }
        for (long i = 0; i < dv; ++i)
            for (long j = 0; j < dk; ++j) Wn[i * dk + j] += bt * r[i] * (real)kt[j];
    }
    /* reverse */
    for (long i = 0; i < n; ++i) G[i] = dstate_out ? (real)dstate_out[st(b, h, H, dv, dk) + i] : (real)0;
    for (long t = T - 1; t >= 0; --t) {
        const real *Wp = Ws + t * n;
        const double *kt = k + tok(b, t, h, T, H, dk);
        const double *qt = q + tok(b, t, h, T, H, dk);
        const double *vt = v + tok(b, t, h, T, H, dv);
        const double *yt = dout + tok(b, t, h, T, H, dv);
        const real bt = (real)beta[tok(b, t, h, T, H, 1)];
        /* recompute this token's forward quantities from W_{t-1} */
        for (long i = 0; i < n; ++i) Wt[i] = Wp[i];
        if (variant == ORACLE_GATED_DELTANET || variant == ORACLE_GATED_DELTANET2) {
            const real a = (real)alpha[tok(b, t, h, T, H, 1)];
            for (long i = 0; i < n; ++i) Wt[i] = a * Wt[i];
        } else if (variant == ORACLE_KIMI_DELTA) {
            const double *at = alpha + tok(b, t, h, T, H, dk);
            for (long i = 0; i < dv; ++i)
                for (long j = 0; j < dk; ++j) Wt[i * dk + j] = Wt[i * dk + j] * (real)at[j];
        }
        /* Wt holds W~ here */
        for (long j = 0; j < dk; ++j) kk[j] = (real)kt[j];
        for (long i = 0; i < dv; ++i) z[i] = (real)vt[i];
        if (variant == ORACLE_GATED_DELTANET2) {
            const double *bt_ = erase_b + tok(b, t, h, T, H, dk);
            const double *wt_ = write_w + tok(b, t, h, T, H, dv);
            for (long j = 0; j < dk; ++j) kk[j] = (real)bt_[j] * kk[j];
            for (long i = 0; i < dv; ++i) z[i] = (real)wt_[i] * z[i];
        }
        for (long i = 0; i < dv; ++i) {
            real pred = 0;
            for (long j = 0; j < dk; ++j) pred += Wt[i * dk + j] * kk[j];
            r[i] = z[i] - pred;
        }
        /* the read: G += dout q^T, dq = W_t^T dout (W_t = W~ + beta r k^T) */
        for (long i = 0; i < dv; ++i)
            for (long j = 0; j < dk; ++j) G[i * dk + j] += (real)yt[i] * (real)qt[j];
        double *dqt = dq + tok(b, t, h, T, H, dk);
        for (long j = 0; j < dk; ++j) {
            real acc = 0;
            for (long i = 0; i < dv; ++i) acc += (Wt[i * dk + j] + bt * r[i] * (real)kt[j]) * (real)yt[i];
            dqt[j] = (double)acc;
        }
        /* the write */
        real dbt = 0;
        for (long i = 0; i < dv; ++i) {
            real acc = 0;
            for (long j = 0; j < dk; ++j) acc += G[i * dk + j] * (real)kt[j];
            g[i] = acc;
            dbt += r[i] * acc;
        }
        dbeta[tok(b, t, h, T, H, 1)] = (double)dbt;
        double *dvt = dvg + tok(b, t, h, T, H, dv);
        for (long i = 0; i < dv; ++i) {
            const real dzi = bt * g[i];
            if (variant == ORACLE_GATED_DELTANET2) {
                dvt[i] = (double)((real)write_w[tok(b, t, h, T, H, dv) + i] * dzi);
                dwrite_w[tok(b, t, h, T, H, dv) + i] = (double)((real)vt[i] * dzi);
            } else {
                dvt[i] = (double)dzi;
            }
        }
        double *dkt = dkg + tok(b, t, h, T, H, dk);
        for (long j = 0; j < dk; ++j) {
            real acc = 0, acc2 = 0;
            for (long i = 0; i < dv; ++i) {
                acc += G[i * dk + j] * r[i];
                acc2 += Wt[i * dk + j] * g[i];
            }
            dkk[j] = -bt * acc2;
            dkt[j] = (double)(bt * acc);
        }
        if (variant == ORACLE_GATED_DELTANET2) {
            const double *bt_ = erase_b + tok(b, t, h, T, H, dk);
            for (long j = 0; j < dk; ++j) {
                dkt[j] += (double)((real)bt_[j] * dkk[j]);
                derase_b[tok(b, t, h, T, H, dk) + j] = (double)((real)kt[j] * dkk[j]);
            }
        } else {
            for (long j = 0; j < dk; ++j) dkt[j] += (double)dkk[j];
        }
        /* dW~ = G - beta g kk^T, into G */
        for (long i = 0; i < dv; ++i)
            for (long j = 0; j < dk; ++j) G[i * dk + j] -= bt * g[i] * kk[j];
        /* the decay */
        if (variant == ORACLE_GATED_DELTANET || variant == ORACLE_GATED_DELTANET2) {
            const real a = (real)alpha[tok(b, t, h, T, H, 1)];
            real acc = 0;
            for (long i = 0; i < n; ++i) acc += G[i] * Wp[i];
            dalpha[tok(b, t, h, T, H, 1)] = (double)acc;
            for (long i = 0; i < n; ++i) G[i] = a * G[i];
        } else if (variant == ORACLE_KIMI_DELTA) {
            const double *at = alpha + tok(b, t, h, T, H, dk);
            double *dat = dalpha + tok(b, t, h, T, H, dk);
            for (long j = 0; j < dk; ++j) {
                real acc = 0;
                for (long i = 0; i < dv; ++i) acc += G[i * dk + j] * Wp[i * dk + j];
                dat[j] = (double)acc;
            }
            for (long i = 0; i < dv; ++i)
                for (long j = 0; j < dk; ++j) G[i * dk + j] = G[i * dk + j] * (real)at[j];
        }
    }
    if (dstate_in)
        for (long i = 0; i < n; ++i) dstate_in[st(b, h, H, dv, dk) + i] = (double)G[i];
}

/*
 * oracle_delta_backward: gradients of L = sum <dout, out> + <dstate_out,
 * state_out> for the forward of oracle_delta_forward (same input layouts).
 * dout [B,T,H,dv] required; dstate_out [B,H,dv,dk] or NULL (zero).  Outputs:
 * dq, dk [B,T,H,dk]; dv [B,T,H,dv]; dbeta [B,T,H]; dalpha like alpha (NULL
 * for DeltaNet); derase_b, dwrite_w like erase_b, write_w (Gated DeltaNet-2
 * only); dstate_in [B,H,dv,dk] or NULL.  Returns 0, or -1 on a bad argument.
 */
int oracle_delta_backward(int variant, long B, long T, long H, long dk, long dv,
                          const double *q, const double *k, const double *v,
                          const double *alpha, const double *erase_b,
                          const double *write_w, const double *beta,
                          const double *state_in, const double *dout,
                          const double *dstate_out, double *dq, double *dkg,
                          double *dvg, double *dalpha, double *derase_b,
                          double *dwrite_w, double *dbeta, double *dstate_in,
                          int nthreads) {
    if (variant < ORACLE_DELTANET || variant > ORACLE_GATED_DELTANET2) return -1;
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    if (!q || !k || !v || !beta || !dout || !dq || !dkg || !dvg || !dbeta) return -1;
    if (variant != ORACLE_DELTANET && (!alpha || !dalpha)) return -1;
    if (variant == ORACLE_GATED_DELTANET2 && (!erase_b || !write_w || !derase_b || !dwrite_w)) return -1;
    const long chains = B * H;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : omp_get_max_threads()) \
    reduction(| : failed)
    for (long c = 0; c < chains; ++c) {
        const size_t n = (size_t)(dv * dk);
        real *buf = (real *)malloc(sizeof(real) * ((size_t)(T + 1) * n + 2 * n + 3 * (size_t)dk + 3 * (size_t)dv));
        if (!buf) { failed = 1; continue; }
        real *Ws = buf, *Wt = Ws + (size_t)(T + 1) * n, *G = Wt + n, *kk = G + n, *z = kk + dk, *r = z + dv,
             *g = r + dv, *dkk = g + dv;
        delta_chain_bwd(variant, c / H, c % H, T, H, dk, dv, q, k, v, alpha, erase_b, write_w, beta,
                        state_in, dout, dstate_out, dq, dkg, dvg, dalpha, derase_b, dwrite_w, dbeta,
                        dstate_in, Ws, Wt, G, kk, z, r, g, dkk);
        free(buf);
    }
    return failed ? -1 : 0;
}

/* ELU(x) + 1 with ELU's scale 1: x + 1 for x > 0, exp(x) otherwise
 * ([VLA] section 2.3, the feature map of keys and queries). */
static real elu_plus_one(real x) { return x > 0 ? x + (real)1 : (real)exp((double)x); }

/*
 * VLA, one (b, h) chain.  Per token, in the order of [VLA] section 2.3:
 *   features   k-hat = phi(k)/|phi(k)|, q-hat = phi(q)/|phi(q)|, phi = ELU+1
 *   rule 1     z = A p;  A <- A - z z^T / (1 + p^T z)     (Sherman-Morrison
 *              for M_t = M_{t-1} + p p^T, section 2.2)
 *   rule 2     a = A k-hat;  alpha-hat = a / |a|
 *   rule 3     S <- S + (v - S k-hat) alpha-hat^T
 *   read       y = S q-hat
 */
static void vla_chain(long b, long h, long T, long H, long d, const double *q,
                      const double *k, const double *v, const double *p,
                      const double *A_in, const double *S_in, double *out,
                      double *A_out, double *S_out, double *khat_out,
                      double *qhat_out, double *ahat_out, double *den_out,
                      real *A, real *S, real *kh, real *qh, real *pp, real *z,
                      real *a, real *r) {
    const size_t s0 = st(b, h, H, d, d);
    for (long i = 0; i < d; ++i)
        for (long j = 0; j < d; ++j) {
            A[i * d + j] = A_in ? (real)A_in[s0 + i * d + j] : (real)(i == j);
            S[i * d + j] = S_in ? (real)S_in[s0 + i * d + j] : (real)0;
        }

    for (long t = 0; t < T; ++t) {
        const size_t o = tok(b, t, h, T, H, d);
        /* feature maps and unit normalisation */
        real nk = 0, nq = 0;
        for (long j = 0; j < d; ++j) {
            kh[j] = elu_plus_one((real)k[o + j]);
            qh[j] = elu_plus_one((real)q[o + j]);
            nk += kh[j] * kh[j];
            nq += qh[j] * qh[j];
        }
        nk = (real)sqrt((double)nk);
        nq = (real)sqrt((double)nq);
        for (long j = 0; j < d; ++j) {
            kh[j] /= nk;
            qh[j] /= nq;
            pp[j] = (real)p[o + j];
        }

        /* rule 1: Sherman-Morrison downdate of the inverse penalty */
        real den = 1;
        for (long i = 0; i < d; ++i) {
            real acc = 0;
            for (long j = 0; j < d; ++j) acc += A[i * d + j] * pp[j];
            z[i] = acc;
        }
        for (long i = 0; i < d; ++i) den += pp[i] * z[i];
        for (long i = 0; i < d; ++i)
            for (long j = 0; j < d; ++j) A[i * d + j] -= z[i] * z[j] / den;

        /* rule 2: gating vector */
        real na = 0;
        for (long i = 0; i < d; ++i) {
            real acc = 0;
            for (long j = 0; j < d; ++j) acc += A[i * d + j] * kh[j];
            a[i] = acc;
            na += acc * acc;
        }
        na = (real)sqrt((double)na);
        for (long i = 0; i < d; ++i) a[i] /= na;

        /* rule 3: residual write along alpha-hat */
        for (long i = 0; i < d; ++i) {
            real acc = 0;
            for (long j = 0; j < d; ++j) acc += S[i * d + j] * kh[j];
            r[i] = (real)v[o + i] - acc;
        }
        for (long i = 0; i < d; ++i)
            for (long j = 0; j < d; ++j) S[i * d + j] += r[i] * a[j];

        /* read */
        for (long i = 0; i < d; ++i) {
            real acc = 0;
            for (long j = 0; j < d; ++j) acc += S[i * d + j] * qh[j];
            out[o + i] = (double)acc;
        }
        if (khat_out) for (long j = 0; j < d; ++j) khat_out[o + j] = (double)kh[j];
        if (qhat_out) for (long j = 0; j < d; ++j) qhat_out[o + j] = (double)qh[j];
        if (ahat_out) for (long j = 0; j < d; ++j) ahat_out[o + j] = (double)a[j];
        if (den_out) den_out[tok(b, t, h, T, H, 1)] = (double)den;
    }
    if (A_out) for (long i = 0; i < d * d; ++i) A_out[s0 + i] = (double)A[i];
    if (S_out) for (long i = 0; i < d * d; ++i) S_out[s0 + i] = (double)S[i];
}

/*
 * VLA with the output read as a ratio of two recurrences, one (b, h) chain
 * ([VLA] section 2.3: the output is a ratio of recurrences as in standard
 * linear attention).  In linear attention the numerator and the denominator
 * accumulate the same way, the denominator over a value of 1; here the
 * denominator is a d-vector n that follows rule 3 with the value 1
 * (reading X7), and the read divides:
 *   rules 1-2  as vla_chain
 *   rule 3     S <- S + (v - S k-hat) alpha-hat^T,
 *              n <- n + (1 - n . k-hat) alpha-hat
 *   read       y = (S q-hat) / (n . q-hat)
 * The steps are written out again here rather than shared with vla_chain.
 */
static void vla_ratio_chain(long b, long h, long T, long H, long d, const double *q,
                            const double *k, const double *v, const double *p,
                            const double *A_in, const double *S_in, const double *n_in,
                            double *out, double *A_out, double *S_out, double *n_out,
                            real *A, real *S, real *n, real *kh, real *qh, real *pp,
                            real *z, real *a, real *r) {
    const size_t s0 = st(b, h, H, d, d), n0 = st(b, h, H, d, 1);
    for (long i = 0; i < d; ++i) {
        for (long j = 0; j < d; ++j) {
            A[i * d + j] = A_in ? (real)A_in[s0 + i * d + j] : (real)(i == j);
            S[i * d + j] = S_in ? (real)S_in[s0 + i * d + j] : (real)0;
        }
        n[i] = n_in ? (real)n_in[n0 + i] : (real)0;
    }
    for (long t = 0; t < T; ++t) {
        const size_t o = tok(b, t, h, T, H, d);
        real nk = 0, nq = 0;
        for (long j = 0; j < d; ++j) {
            kh[j] = elu_plus_one((real)k[o + j]);
            qh[j] = elu_plus_one((real)q[o + j]);
            nk += kh[j] * kh[j];
            nq += qh[j] * qh[j];
        }
        nk = (real)sqrt((double)nk);
        nq = (real)sqrt((double)nq);
        for (long j = 0; j < d; ++j) {
            kh[j] /= nk;
            qh[j] /= nq;
            pp[j] = (real)p[o + j];
        }
        /* rule 1 */
        real den = 1;
        for (long i = 0; i < d; ++i) {
            real acc = 0;
            for (long j = 0; j < d; ++j) acc += A[i * d + j] * pp[j];
            z[i] = acc;
        }
        for (long i = 0; i < d; ++i) den += pp[i] * z[i];
        for (long i = 0; i < d; ++i)
            for (long j = 0; j < d; ++j) A[i * d + j] -= z[i] * z[j] / den;
        /* rule 2 */
        real na = 0;
        for (long i = 0; i < d; ++i) {
            real acc = 0;
            for (long j = 0; j < d; ++j) acc += A[i * d + j] * kh[j];
            a[i] = acc;
            na += acc * acc;
        }
        na = (real)sqrt((double)na);
        for (long i = 0; i < d; ++i) a[i] /= na;
        /* rule 3, for the values and for the constant 1 */
        for (long i = 0; i < d; ++i) {
            real acc = 0;
            for (long j = 0; j < d; ++j) acc += S[i * d + j] * kh[j];
            r[i] = (real)v[o + i] - acc;
        }
        for (long i = 0; i < d; ++i)
            for (long j = 0; j < d; ++j) S[i * d + j] += r[i] * a[j];
        real rn = 1;
        for (long j = 0; j < d; ++j) rn -= n[j] * kh[j];
        for (long j = 0; j < d; ++j) n[j] += rn * a[j];
        /* read: the ratio */
        real dq = 0;
        for (long j = 0; j < d; ++j) dq += n[j] * qh[j];
        for (long i = 0; i < d; ++i) {
            real acc = 0;
            for (long j = 0; j < d; ++j) acc += S[i * d + j] * qh[j];
            out[o + i] = (double)(acc / dq);
        }
    }
    if (A_out) for (long i = 0; i < d * d; ++i) A_out[s0 + i] = (double)A[i];
    if (S_out) for (long i = 0; i < d * d; ++i) S_out[s0 + i] = (double)S[i];
    if (n_out) for (long i = 0; i < d; ++i) n_out[n0 + i] = (double)n[i];
}

/*
 * oracle_vla_forward_ratio: VLA with the ratio read over a [B,T] block.
 * Layouts as oracle_vla_forward, plus the denominator state n_in / n_out
 * [B,H,d] (NULL n_in = zero, NULL n_out = not written).
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_vla_forward_ratio(long B, long T, long H, long d, const double *q,
                             const double *k, const double *v, const double *p,
                             const double *A_in, const double *S_in, const double *n_in,
                             double *out, double *A_out, double *S_out, double *n_out,
                             int nthreads) {
    if (B < 0 || T < 0 || H < 0 || d <= 0) return -1;
    if (!q || !k || !v || !p || !out) return -1;
    const long chains = B * H;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : omp_get_max_threads()) \
    reduction(| : failed)
    for (long c = 0; c < chains; ++c) {
        real *buf = (real *)malloc(sizeof(real) * (size_t)(2 * d * d + 7 * d));
        if (!buf) { failed = 1; continue; }
        real *A = buf, *S = buf + d * d, *w = buf + 2 * d * d;
        vla_ratio_chain(c / H, c % H, T, H, d, q, k, v, p, A_in, S_in, n_in, out, A_out, S_out,
                        n_out, A, S, w, w + d, w + 2 * d, w + 3 * d, w + 4 * d, w + 5 * d, w + 6 * d);
        free(buf);
    }
    return failed ? -1 : 0;
}

/*
 * oracle_vla_forward: VLA over a [B,T] block, dk = dv = d.
 * Layouts: q, k, v, p, out [B,T,H,d]; A_in/A_out/S_in/S_out [B,H,d,d]
 * (NULL A_in = identity, NULL S_in = zero, NULL outs = not written).
 * Optional per-token diagnostics [B,T,H,d]: k-hat, q-hat, alpha-hat; and the
 * Sherman-Morrison denominator 1 + p^T z as [B,T,H].
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_vla_forward(long B, long T, long H, long d, const double *q,
                       const double *k, const double *v, const double *p,
                       const double *A_in, const double *S_in, double *out,
                       double *A_out, double *S_out, double *khat_out,
                       double *qhat_out, double *ahat_out, double *den_out,
                       int nthreads) {
    if (B < 0 || T < 0 || H < 0 || d <= 0) return -1;
    if (!q || !k || !v || !p || !out) return -1;
    const long chains = B * H;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : omp_get_max_threads()) \
    reduction(| : failed)
    for (long c = 0; c < chains; ++c) {
        real *buf = (real *)malloc(sizeof(real) * (size_t)(2 * d * d + 6 * d));
        if (!buf) { failed = 1; continue; }
        real *A = buf, *S = buf + d * d, *w = buf + 2 * d * d;
        vla_chain(c / H, c % H, T, H, d, q, k, v, p, A_in, S_in, out, A_out, S_out,
                  khat_out, qhat_out, ahat_out, den_out, A, S, w, w + d, w + 2 * d,
                  w + 3 * d, w + 4 * d, w + 5 * d);
        free(buf);
    }
    return failed ? -1 : 0;
}

/*
 * Log-linear (Fenwick-tree) readout of the delta-rule family, one (b, h)
 * chain ("Technical summary: adaptive memory decay for log-linear
 * attention", "Problem definition": the memory is a Fenwick-tree hierarchy
 * of O(log T) levels and each step's output is the lambda^(l)_t-weighted sum
 * of the levels' reads).
 *
 * Readings (the page gives neither the partition nor how the levels evolve):
 *   - levels follow the Fenwick partition of the prefix: for the query at
 *     absolute position t, token t itself is level 0 and an earlier token s is
 *     level msb(t xor s) + 1 (the lowbit segments of [0, t), level l holding
 *     2^(l-1) tokens);
 *   - every level's memory takes the variant's transition each step (decay,
 *     then the delta rule's erase along e with that level's own prediction:
 *     S <- S~ - beta (S~ e) k^T), and only level 0 receives the new write
 *     beta z k^T; so the levels sum to exactly the single memory W of the
 *     plain scan, and lambda = 1 on every level gives the plain scan's output;
 *   - moving to position t >= 1, levels 0 .. ctz(t) merge into level
 *     ctz(t) + 1 (the segment of the last 2^ctz(t) tokens), leaving levels
 *     1 .. ctz(t) empty.
 * Per token, in this order: merge, transition of every level, write to
 * level 0, read y = sum_l lambda_l S_l q.
 * Levels: nL of them, S[l] at W + l*dv*dk; t0 is the absolute position of
 * token 0 (the levels in state_in are those after position t0 - 1).
 */
static void loglin_chain(int variant, long b, long h, long T, long H, long dk, long dv, long nL,
                         long t0, const double *q, const double *k, const double *v,
                         const double *alpha, const double *erase_b, const double *write_w,
                         const double *beta, const double *lam, const double *state_in,
                         double *out, double *state_out, real *W, real *kk, real *target) {
    const size_t lsz = (size_t)dv * dk;
    const size_t sbase = st(b, h, H, nL * dv, dk);  /* [B,H,nL,dv,dk] */
    for (size_t i = 0; i < (size_t)nL * lsz; ++i)
        W[i] = state_in ? (real)state_in[sbase + i] : (real)0;

    for (long t = 0; t < T; ++t) {
        const long pos = t0 + t;
        const double *kt = k + tok(b, t, h, T, H, dk);
        const double *qt = q + tok(b, t, h, T, H, dk);
        const double *vt = v + tok(b, t, h, T, H, dv);
        const double *lt = lam + tok(b, t, h, T, H, nL);
        const real bt = (real)beta[tok(b, t, h, T, H, 1)];

        /* Fenwick merge: levels 0..p into level p+1, p = ctz(pos) */
        if (pos > 0) {
            long p = 0;
            while (((pos >> p) & 1) == 0) ++p;
            real *dst = W + (size_t)(p + 1) * lsz;
            for (long l = 0; l <= p; ++l) {
                real *src = W + (size_t)l * lsz;
                for (size_t i = 0; i < lsz; ++i) { dst[i] += src[i]; src[i] = 0; }
            }
        }

        /* read key and write target */
        for (long j = 0; j < dk; ++j) kk[j] = (real)kt[j];
        for (long i = 0; i < dv; ++i) target[i] = (real)vt[i];
        if (variant == ORACLE_GATED_DELTANET2) {
            const double *eb = erase_b + tok(b, t, h, T, H, dk);
            const double *ww = write_w + tok(b, t, h, T, H, dv);
            for (long j = 0; j < dk; ++j) kk[j] = (real)eb[j] * kk[j];
            for (long i = 0; i < dv; ++i) target[i] = (real)ww[i] * target[i];
        }

        /* transition of every level: decay, then erase with its own prediction */
        for (long l = 0; l < nL; ++l) {
            real *S = W + (size_t)l * lsz;
            if (variant == ORACLE_GATED_DELTANET || variant == ORACLE_GATED_DELTANET2) {
                const real a = (real)alpha[tok(b, t, h, T, H, 1)];
                for (size_t i = 0; i < lsz; ++i) S[i] = a * S[i];
            } else if (variant == ORACLE_KIMI_DELTA) {
                const double *at = alpha + tok(b, t, h, T, H, dk);
                for (long i = 0; i < dv; ++i)
                    for (long j = 0; j < dk; ++j) S[i * dk + j] = S[i * dk + j] * (real)at[j];
            }
            for (long i = 0; i < dv; ++i) {
                real pred = 0;
                for (long j = 0; j < dk; ++j) pred += S[i * dk + j] * kk[j];
                for (long j = 0; j < dk; ++j) S[i * dk + j] -= bt * pred * (real)kt[j];
            }
        }

        /* the new write goes to level 0 */
        for (long i = 0; i < dv; ++i)
            for (long j = 0; j < dk; ++j) W[i * dk + j] += bt * target[i] * (real)kt[j];

        /* lambda-weighted read of the levels */
        double *yt = out + tok(b, t, h, T, H, dv);
        for (long i = 0; i < dv; ++i) {
            real acc = 0;
            for (long l = 0; l < nL; ++l) {
                const real *S = W + (size_t)l * lsz;
                real r = 0;
                for (long j = 0; j < dk; ++j) r += S[i * dk + j] * (real)qt[j];
                acc += (real)lt[l] * r;
            }
            yt[i] = (double)acc;
        }
    }
    if (state_out)
        for (size_t i = 0; i < (size_t)nL * lsz; ++i) state_out[sbase + i] = (double)W[i];
}

/*
 * oracle_loglinear_forward: the log-linear readout over a [B,T] block.
 * Layouts as oracle_delta_forward; lam [B,T,H,nL]; state_in / state_out
 * [B,H,nL,dv,dk] (NULL in = every level empty).  The caller must give enough
 * levels: nL >= floor(log2(t0 + T - 1)) + 2 when t0 + T >= 2 (else -1).
 */
int oracle_loglinear_forward(int variant, long B, long T, long H, long dk, long dv, long nL,
                             long t0, const double *q, const double *k, const double *v,
                             const double *alpha, const double *erase_b,
                             const double *write_w, const double *beta, const double *lam,
                             const double *state_in, double *out, double *state_out,
                             int nthreads) {
    if (variant < ORACLE_DELTANET || variant > ORACLE_GATED_DELTANET2) return -1;
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0 || nL <= 0 || t0 < 0) return -1;
    if (!q || !k || !v || !beta || !lam || !out) return -1;
    if (variant != ORACLE_DELTANET && !alpha) return -1;
    if (variant == ORACLE_GATED_DELTANET2 && (!erase_b || !write_w)) return -1;
    const long last = t0 + T - 1;
    if (last >= 1) {
        long need = 1;
        while ((1L << (need - 1)) <= last) ++need;  /* floor(log2(last)) + 2 */
        if (nL < need) return -1;
    }
    const long chains = B * H;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : omp_get_max_threads()) \
    reduction(| : failed)
    for (long c = 0; c < chains; ++c) {
        real *buf = (real *)malloc(sizeof(real) * (size_t)(nL * dv * dk + dk + dv));
        if (!buf) { failed = 1; continue; }
        loglin_chain(variant, c / H, c % H, T, H, dk, dv, nL, t0, q, k, v, alpha, erase_b, write_w,
                     beta, lam, state_in, out, state_out, buf, buf + nL * dv * dk,
                     buf + nL * dv * dk + dk);
        free(buf);
    }
    return failed ? -1 : 0;
}

/* Size of `real` as compiled (8 for the fp64 oracle, 4 for the spread check). */
int oracle_real_bytes(void) { return (int)sizeof(real); }
