"""Test-only float64 numpy model of the chunkwise-parallel scan.

This is the algebra the HIP kernels evaluate, written out plainly so that the
CPU tier can check it against the token-by-token oracle before any kernel is
trusted.  It is derived from the per-token rules (linear-attention
architectures page, "Technical details"; VLA page, section 2.3) and shares no
code with the oracle or with the HIP library.

Per chunk of C tokens (rows = tokens, S = state at the chunk start, dv x dk):

Gated DeltaNet (DeltaNet: every alpha = 1), gamma_t = prod_{j<=t} alpha_j:
    L     = strict_tril(diag(beta) (K K^T * Gamma)),  Gamma_ts = gamma_t/gamma_s
    U     = (I + L)^-1 (diag(beta) V - diag(beta gamma) K S^T)
    Y     = diag(gamma) Q S^T + (tril(Q K^T) * Gamma) U
    S'    = gamma_C S + U^T diag(gamma_C / gamma) K
Gated DeltaNet-2: L from E K^T (e_t . k_s), V -> Z and K S^T -> E S^T in U.
Kimi Delta (g_t = prod_{j<=t} alpha_j per key channel):
    L_ts  = beta_t sum_c k_tc k_sc g_tc/g_sc  (s < t)
    U     = (I + L)^-1 diag(beta) (V - (K*G) S^T)
    Y     = (Q*G) S^T + Aqk U,  Aqk_ts = sum_c q_tc k_sc g_tc/g_sc  (s <= t)
    S'    = S diag(g_C) + U^T (K * g_C/G)
VLA state (read key k-hat, write key alpha-hat):
    U     = (I + strict_tril(Khat Ahat^T))^-1 (V - Khat S^T)
    Y     = Qhat S^T + tril(Qhat Ahat^T) U
    S'    = S + U^T Ahat
VLA inverse penalty (A_c = inverse penalty at the chunk start):
    I + P A_c P^T = L D L^T,  Z = L^-1 P A_c   (row t: z_t = A_{t-1} p_t)
    A_t khat_t = A_c khat_t - sum_{s<=t} z_s (z_s . khat_t) / D_s
    A_next = A_c - Z^T D^-1 Z
"""
from __future__ import annotations

import numpy as np


def _phi(x):
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def delta_chunked(variant, q, k, v, beta, alpha=None, erase_b=None, write_w=None,
                  state_in=None, C=64):
    B, T, H, dk = q.shape
    dv = v.shape[3]
    out = np.zeros((B, T, H, dv))
    state_out = np.zeros((B, H, dv, dk))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dv, dk)) if state_in is None else state_in[b, h].copy()
            for c0 in range(0, T, C):
                c1 = min(T, c0 + C)
                n = c1 - c0
                Q, K, V = q[b, c0:c1, h], k[b, c0:c1, h], v[b, c0:c1, h]
                be = beta[b, c0:c1, h]
                tril = np.tril(np.ones((n, n)))
                stril = np.tril(np.ones((n, n)), -1)
                if variant == "kda":
                    lg = np.cumsum(np.log(alpha[b, c0:c1, h]), axis=0)      # [n, dk]
                    # Gamma per channel: exp(G_t - G_s), evaluated only for s <= t
                    D = lg[:, None, :] - lg[None, :, :]                      # [t, s, c]
                    D = np.where(tril[:, :, None] > 0, D, -np.inf)
                    Gm = np.exp(D)
                    Akk = np.einsum("tc,sc,tsc->ts", K, K, Gm)
                    Aqk = np.einsum("tc,sc,tsc->ts", Q, K, Gm)
                    G = np.exp(lg)
                    L = stril * (be[:, None] * Akk)
                    rhs = be[:, None] * (V - (K * G) @ S.T)
                    U = np.linalg.solve(np.eye(n) + L, rhs)
                    Y = (Q * G) @ S.T + (Aqk * tril) @ U
                    S = S * G[-1][None, :] + U.T @ (K * np.exp(lg[-1][None, :] - lg))
                else:
                    if variant == "deltanet":
                        lg = np.zeros(n)
                    else:
                        lg = np.cumsum(np.log(alpha[b, c0:c1, h]))
                    D = lg[:, None] - lg[None, :]
                    Gam = np.where(tril > 0, np.exp(np.where(tril > 0, D, 0.0)), 0.0)
                    g = np.exp(lg)
                    if variant == "gdn2":
                        E = erase_b[b, c0:c1, h] * K
                        Z = write_w[b, c0:c1, h] * V
                    else:
                        E, Z = K, V
                    L = stril * (be[:, None] * (E @ K.T) * Gam)
                    rhs = be[:, None] * Z - (be * g)[:, None] * (E @ S.T)
                    U = np.linalg.solve(np.eye(n) + L, rhs)
                    Y = g[:, None] * (Q @ S.T) + ((Q @ K.T) * Gam) @ U
                    S = g[-1] * S + U.T @ (np.exp(lg[-1] - lg)[:, None] * K)
                out[b, c0:c1, h] = Y
            state_out[b, h] = S
    return out, state_out


def kda_blocks_by_levels(K, Q, lg):
    """Kimi Delta's two decayed Gram blocks of one 16-token chunk, formed the
    way the chunked kernel's exact path forms them: entry (t, s), s < t, at
    level b = highest set bit of t ^ s, with both factors taken against the
    reference token m = (t & ~(2b - 1)) + b - 1 (so s <= m < t and each factor
    is at most 1); the diagonal of Aqk undecayed.  lg: [16, dk] running log
    decay.  Returns (Akk, Aqk) with Akk_ts = sum_c k_tc k_sc exp(lg_tc - lg_sc)
    for s < t (zero elsewhere) and Aqk_ts the same with q_t, for s <= t."""
    n = K.shape[0]
    assert n == 16
    Akk = np.zeros((n, n))
    Aqk = np.zeros((n, n))
    for b in (8, 4, 2, 1):
        rows = np.zeros((n, K.shape[1]))   # exp(lg_t - lg_m) for t in the upper half of its block
        cols = np.zeros((n, K.shape[1]))   # exp(lg_m - lg_s) for s in the lower half
        for t in range(n):
            m = (t & ~(2 * b - 1)) + b - 1
            if t & b:
                rows[t] = np.exp(lg[t] - lg[m])
            else:
                cols[t] = np.exp(lg[m] - lg[t])
        assert rows.max(initial=0) <= 1 and cols.max(initial=0) <= 1
        gk = (K * rows) @ (K * cols).T
        gq = (Q * rows) @ (K * cols).T
        for t in range(n):
            for s in range(n):
                x = t ^ s
                if b <= x < 2 * b and t & b:
                    Akk[t, s] = gk[t, s]
                    Aqk[t, s] = gq[t, s]
    Aqk[np.diag_indices(n)] = np.sum(Q * K, axis=1)
    return Akk, Aqk


def vla_chunked(q, k, v, p, A_in=None, S_in=None, C=64):
    B, T, H, d = q.shape
    out = np.zeros((B, T, H, d))
    A_out = np.zeros((B, H, d, d))
    S_out = np.zeros((B, H, d, d))
    for b in range(B):
        for h in range(H):
            A = np.eye(d) if A_in is None else A_in[b, h].copy()
            S = np.zeros((d, d)) if S_in is None else S_in[b, h].copy()
            for c0 in range(0, T, C):
                c1 = min(T, c0 + C)
                n = c1 - c0
                fk = _phi(k[b, c0:c1, h])
                fq = _phi(q[b, c0:c1, h])
                Kh = fk / np.linalg.norm(fk, axis=1, keepdims=True)
                Qh = fq / np.linalg.norm(fq, axis=1, keepdims=True)
                P = p[b, c0:c1, h]
                V = v[b, c0:c1, h]
                # inverse penalty: LDL^T of I + P A P^T via Cholesky
                R = np.linalg.cholesky(np.eye(n) + P @ A @ P.T)
                Dg = np.diag(R) ** 2
                Lu = R / np.diag(R)[None, :]
                Z = np.linalg.solve(Lu, P @ A)
                AK = Kh @ A - np.tril((Kh @ Z.T) / Dg[None, :]) @ Z
                Ah = AK / np.linalg.norm(AK, axis=1, keepdims=True)
                A = A - Z.T @ (Z / Dg[:, None])
                # state
                stril = np.tril(np.ones((n, n)), -1)
                U = np.linalg.solve(np.eye(n) + stril * (Kh @ Ah.T), V - Kh @ S.T)
                Y = Qh @ S.T + (np.tril(np.ones((n, n))) * (Qh @ Ah.T)) @ U
                S = S + U.T @ Ah
                out[b, c0:c1, h] = Y
            A_out[b, h] = A
            S_out[b, h] = S
    return out, A_out, S_out


def kda_paired(q, k, v, beta, alpha, state_in=None):
    """Kimi Delta stepped over pairs of 16-token sub-chunks, in the form the
    chunked kernel evaluates: each sub-chunk's tiles are formed locally (its
    own running decay), then made relative to the pair (the odd sub-chunk's
    K*G and Q*G times the even one's end decay g0, the even one's K*gC/G
    times the odd one's g1), both sub-chunks act on the state at the pair
    start, and they are coupled by the cross blocks
        G10 = (K1*G1)(K0*g0/G0)^T,  A10 = (Q1*G1)(K0*g0/G0)^T,
        U0 = T00 (V0 - Z0),  U1 = T11 (V1 - Z1) - T11 G10 U0,
    with Tii = (I + Lii)^-1 diag(beta_i).  A ragged tail is padded with zero
    keys, queries and values, decay 1 and beta 0."""
    B, T, H, dk = q.shape
    dv = v.shape[3]
    n2 = -(-T // 32) * 32
    pad = lambda x, fill: np.concatenate([x, np.full((x.shape[0], n2 - T) + x.shape[2:], fill)], axis=1)
    q, k, v, beta, alpha = pad(q, 0.0), pad(k, 0.0), pad(v, 0.0), pad(beta, 0.0), pad(alpha, 1.0)
    out = np.zeros((B, n2, H, dv))
    state_out = np.zeros((B, H, dv, dk))
    tril = np.tril(np.ones((16, 16)))
    stril = np.tril(np.ones((16, 16)), -1)

    def local(t0, b, h):
        K, Q, V = k[b, t0:t0 + 16, h], q[b, t0:t0 + 16, h], v[b, t0:t0 + 16, h]
        be = beta[b, t0:t0 + 16, h]
        lg = np.cumsum(np.log(alpha[b, t0:t0 + 16, h]), axis=0)
        D = np.where(tril[:, :, None] > 0, lg[:, None, :] - lg[None, :, :], -np.inf)
        Gm = np.exp(D)
        Akk = np.einsum("tc,sc,tsc->ts", K, K, Gm)
        Aqk = np.einsum("tc,sc,tsc->ts", Q, K, Gm) * tril
        Tm = np.linalg.inv(np.eye(16) + stril * (be[:, None] * Akk)) * be[None, :]
        G = np.exp(lg)
        return dict(kd=K * G, qd=Q * G, ke=K * np.exp(lg[-1] - lg), gc=G[-1], aqk=Aqk, T=Tm, V=V)

    for b in range(B):
        for h in range(H):
            S = np.zeros((dv, dk)) if state_in is None else state_in[b, h].copy()
            for t0 in range(0, n2, 32):
                x0, x1 = local(t0, b, h), local(t0 + 16, b, h)
                G10 = x1["kd"] @ x0["ke"].T
                A10 = x1["qd"] @ x0["ke"].T
                M10 = -x1["T"] @ G10
                kd1, qd1 = x1["kd"] * x0["gc"], x1["qd"] * x0["gc"]
                ke0 = x0["ke"] * x1["gc"]
                U0 = x0["T"] @ (x0["V"] - x0["kd"] @ S.T)
                U1 = x1["T"] @ (x1["V"] - kd1 @ S.T) + M10 @ U0
                out[b, t0:t0 + 16, h] = x0["qd"] @ S.T + x0["aqk"] @ U0
                out[b, t0 + 16:t0 + 32, h] = qd1 @ S.T + A10 @ U0 + x1["aqk"] @ U1
                S = S * (x0["gc"] * x1["gc"])[None, :] + U0.T @ ke0 + U1.T @ x1["ke"]
            state_out[b, h] = S
    return out[:, :T], state_out


def delta_chunked_backward(variant, q, k, v, beta, dout, alpha=None, erase_b=None, write_w=None,
                           state_in=None, dstate_out=None, C=64, dlog_direct=False):
    """Adjoint of the chunked form above for DeltaNet, Gated DeltaNet and
    Gated DeltaNet-2, in the residual form the GPU evaluates: per chunk, with
    N = strict(E K^T * Gam), A = lower(Q K^T * Gam) diag(beta) and
    Kc = diag(beta gamma_C / gamma) K,
        R = (I + N diag(beta))^{-1} (Z - diag(gamma) E S^T),
        Y = diag(gamma) Q S^T + A R,   S' = gamma_C S + R^T Kc,
    and in reverse, from dY and dS':
        dR = A^T dY + Kc dS'^T,   dX = (I + N diag(beta))^{-T} dR,
        dS = gamma_C dS' + dY^T diag(gamma) Q - dX^T diag(gamma) E,
    with every other gradient a product of these chunk operands (written out
    below).  Returns the same dict as oracle.delta_backward."""
    B, T, H, dk = q.shape
    dv = v.shape[3]
    g2 = variant == "gdn2"
    out = {"dq": np.zeros((B, T, H, dk)), "dk": np.zeros((B, T, H, dk)), "dv": np.zeros((B, T, H, dv)),
           "dbeta": np.zeros((B, T, H)), "dstate_in": np.zeros((B, H, dv, dk))}
    if variant != "deltanet":
        out["dalpha"] = np.zeros((B, T, H))
    if g2:
        out["derase_b"] = np.zeros((B, T, H, dk))
        out["dwrite_w"] = np.zeros((B, T, H, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dv, dk)) if state_in is None else state_in[b, h].copy()
            chunks = []
            for c0 in range(0, T, C):               # forward, keeping each chunk's operands
                c1 = min(T, c0 + C)
                n = c1 - c0
                Q, K, V = q[b, c0:c1, h], k[b, c0:c1, h], v[b, c0:c1, h]
                be = beta[b, c0:c1, h]
                tril = np.tril(np.ones((n, n)))
                stril = np.tril(np.ones((n, n)), -1)
                lg = np.zeros(n) if variant == "deltanet" else np.cumsum(np.log(alpha[b, c0:c1, h]))
                Gam = np.where(tril > 0, np.exp(np.where(tril > 0, lg[:, None] - lg[None, :], 0.0)), 0.0)
                g = np.exp(lg)
                E = erase_b[b, c0:c1, h] * K if g2 else K
                Z = write_w[b, c0:c1, h] * V if g2 else V
                Nm = stril * (E @ K.T) * Gam
                Am = tril * (Q @ K.T) * Gam
                M = np.eye(n) + Nm * be[None, :]
                R = np.linalg.solve(M, Z - g[:, None] * (E @ S.T))
                sc = be * np.exp(lg[-1] - lg)
                chunks.append((c0, c1, S.copy(), Q, K, V, E, be, lg, g, Gam, Nm, Am, M, R, sc))
                S = g[-1] * S + R.T @ (sc[:, None] * K)
            dS = np.zeros((dv, dk)) if dstate_out is None else dstate_out[b, h].copy()
            for (c0, c1, S0, Q, K, V, E, be, lg, g, Gam, Nm, Am, M, R, sc) in reversed(chunks):
                n = c1 - c0
                tril = np.tril(np.ones((n, n)))
                stril = np.tril(np.ones((n, n)), -1)
                dY = dout[b, c0:c1, h]
                Kc = sc[:, None] * K
                A = Am * be[None, :]
                dR = A.T @ dY + Kc @ dS.T
                dKc = R @ dS
                dX = np.linalg.solve(M.T, dR)
                dlg = np.zeros(n)
                # S' = gamma_C S + R^T Kc
                dgC = np.sum(dS * S0)
                dSn = g[-1] * dS + (g[:, None] * dY).T @ Q - dX.T @ (g[:, None] * E)
                # Y = diag(g) Q S^T + A R
                dQ = g[:, None] * (dY @ S0)
                dg = np.sum(dY * (Q @ S0.T), axis=1)
                dA = (dY @ R.T) * tril
                dbe = np.sum(dA * Am, axis=0)
                dAm = dA * be[None, :]
                # R = M^{-1} X, X = Z - diag(g) E S^T, M = I + N diag(beta)
                dZ = dX
                dE = -g[:, None] * (dX @ S0)
                dg += -np.sum(dX * (E @ S0.T), axis=1)
                dLp = -(dX @ R.T) * stril
                dbe += np.sum(dLp * Nm, axis=0)
                dNm = dLp * be[None, :]
                # N = strict(E K^T * Gam), Am = lower(Q K^T * Gam)
                dEK = dNm * Gam
                dE += dEK @ K
                dK = dEK.T @ E
                dQK = dAm * Gam
                dQ += dQK @ K
                dK += dQK.T @ Q
                dGam = dNm * (E @ K.T) + dAm * (Q @ K.T)
                # Kc = diag(sc) K, sc = beta exp(lg_C - lg)
                dK += sc[:, None] * dKc
                dsc = np.sum(dKc * K, axis=1)
                dbe += dsc * np.exp(lg[-1] - lg)
                # the decay exponents
                gw = dGam * Gam
                dlg += gw.sum(axis=1) - gw.sum(axis=0)
                dlg += dg * g
                dlg[-1] += dgC * g[-1] + np.sum(dsc * sc)
                dlg -= dsc * sc
                if g2:
                    out["derase_b"][b, c0:c1, h] = K * dE
                    dK += erase_b[b, c0:c1, h] * dE
                    out["dwrite_w"][b, c0:c1, h] = V * dZ
                    out["dv"][b, c0:c1, h] = write_w[b, c0:c1, h] * dZ
                else:
                    dK += dE
                    out["dv"][b, c0:c1, h] = dZ
                out["dq"][b, c0:c1, h] = dQ
                out["dk"][b, c0:c1, h] = dK
                out["dbeta"][b, c0:c1, h] = dbe
                if variant != "deltanet":
                    if dlog_direct:
                        # the same sums with the cancelling terms left out: the
                        # Gamma terms with both indices >= j and the sc terms of
                        # tokens >= j against the last token's sum
                        dg_g = (dg * g)[::-1].cumsum()[::-1]
                        sc_pre = np.concatenate([[0.0], np.cumsum(dsc * sc)[:-1]])
                        dlog = np.array([gw[j:, :j].sum() for j in range(n)]) + dg_g + dgC * g[-1] + sc_pre
                    else:
                        dlog = np.cumsum(dlg[::-1])[::-1]      # d log(alpha_j) = sum_{t >= j} dlg_t
                    out["dalpha"][b, c0:c1, h] = dlog / alpha[b, c0:c1, h]
                dS = dSn
            out["dstate_in"][b, h] = dS
    return out


def delta_record_adjoint(variant, q, k, v, beta, dout, alpha=None, erase_b=None, write_w=None,
                         state_in=None, dstate_out=None, C=16):
    """The reverse scan in the record form the GPU's adjoint kernel runs: per
    chunk, with Tc = (I + N diag(beta))^{-1}, Aq = lower(Q K^T * Gam) diag(beta),
    Ahat = diag(beta gamma_C / gamma) K and Ahat' = Tc^T Ahat,
        dX  = (Aq Tc)^T dY + Ahat' G'^T,
        G^T = gamma_C G'^T + (diag(gamma) Q)^T dY - (diag(gamma) E)^T dX.
    Returns (dX [B, T, H, dv], dstate_in [B, H, dv, dk]); dX is the gradient of
    the targets z (v, or w * v for Gated DeltaNet-2)."""
    B, T, H, dk = q.shape
    dv = v.shape[3]
    g2 = variant == "gdn2"
    dX = np.zeros((B, T, H, dv))
    dS_in = np.zeros((B, H, dv, dk))
    for b in range(B):
        for h in range(H):
            recs = []
            for c0 in range(0, T, C):
                c1 = min(T, c0 + C)
                n = c1 - c0
                Q, K = q[b, c0:c1, h], k[b, c0:c1, h]
                be = beta[b, c0:c1, h]
                tril = np.tril(np.ones((n, n)))
                stril = np.tril(np.ones((n, n)), -1)
                lg = np.zeros(n) if variant == "deltanet" else np.cumsum(np.log(alpha[b, c0:c1, h]))
                Gam = np.where(tril > 0, np.exp(np.where(tril > 0, lg[:, None] - lg[None, :], 0.0)), 0.0)
                g = np.exp(lg)
                E = erase_b[b, c0:c1, h] * K if g2 else K
                Tc = np.linalg.inv(np.eye(n) + (stril * (E @ K.T) * Gam) * be[None, :])
                Aq = (tril * (Q @ K.T) * Gam) * be[None, :]
                Ah = (be * np.exp(lg[-1] - lg))[:, None] * K
                recs.append((c0, c1, Tc.T @ Ah, Aq @ Tc, g[:, None] * Q, g[:, None] * E, g[-1]))
            G = np.zeros((dv, dk)) if dstate_out is None else dstate_out[b, h].copy()
            for (c0, c1, Ap, AqTc, gQ, gE, gC) in reversed(recs):
                dY = dout[b, c0:c1, h]
                x = AqTc.T @ dY + Ap @ G.T
                dX[b, c0:c1, h] = x
                G = (gC * G.T + gQ.T @ dY - gE.T @ x).T
            dS_in[b, h] = G
    return dX, dS_in
