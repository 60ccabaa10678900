"""NumPy fp64 statement of the chunked matrix form used by the HIP kernels.

Test-only.  It restates the per-chunk algebra that the GPU path evaluates, so
that tests can prove it equals the sequential definition (the oracle) before
any kernel result is compared.  It shares no code with either side.

Within a chunk (local tokens t = 0..C-1, weights theta_c and momentum s_in at
the chunk start, gradients g_j at theta_c) unrolling the momentum and write
rules of the Titans pages gives

    theta_t = a_t theta_c - b_t s_in - sum_{j<t} c_{t,j} g_j
    s_C     = p s_in + sum_j w_j g_j

with the column recurrences
    a_{t+1}      = (1 - alpha_t) a_t
    b_{t+1}      = (1 - alpha_t) b_t + eta_t prod_{m<=t} beta_m
    c_{t+1,j}    = (1 - alpha_t) c_{t,j} + eta_t (1 - beta_j) prod_{j<m<=t} beta_m   (j <= t)
    p            = prod_m beta_m,   w_j = (1 - beta_j) prod_{j<m<C} beta_m.
Because every gradient is an outer product delta h^T, reads at the in-chunk
weights become decay-masked "attention-like" products (rows are tokens):
    U_l = diag(a) Hq W_l^T - diag(b) Hq S_l^T - (Cm * Hq Hk^T) Delta_l.
"""
import numpy as np


def _sig(z):
    return 1.0 / (1.0 + np.exp(-z))


def _silu(z):
    return z * _sig(z)


def _silu_p(z):
    s = _sig(z)
    return s * (1.0 + z * (1.0 - s))


def split(theta, widths):
    out, off = [None], 0
    for l in range(1, len(widths)):
        n = widths[l] * widths[l - 1]
        out.append(theta[off:off + n].reshape(widths[l], widths[l - 1]).copy())
        off += n
    return out


def join(mats):
    return np.concatenate([m.reshape(-1) for m in mats[1:]])


def gate_coefficients(al, et, be):
    """a, b (length n+1), Cm (n+1 rows x n cols), p, w for one chunk of n tokens."""
    n = len(al)
    a = np.ones(n + 1)
    b = np.zeros(n + 1)
    Cm = np.zeros((n + 1, n))
    pb = 1.0
    Bb = np.zeros(n)
    for t in range(n):
        pb *= be[t]
        Bb[:t] *= be[t]
        Bb[t] = 1.0
        a[t + 1] = (1 - al[t]) * a[t]
        b[t + 1] = (1 - al[t]) * b[t] + et[t] * pb
        Cm[t + 1] = (1 - al[t]) * Cm[t]
        Cm[t + 1, :t + 1] += et[t] * (1 - be[:t + 1]) * Bb[:t + 1]
    w = (1 - be) * Bb
    return a, b, Cm, pb, w


def chunk_scan_seq(q, k, v, alpha, eta, beta, theta0, s0, C, widths):
    """One sequence: q/k/v [T,d], gates [T], theta0/s0 [P] -> (y, theta_T, s_T)."""
    L = len(widths) - 1
    W, S = split(np.asarray(theta0, float), widths), split(np.asarray(s0, float), widths)
    T = q.shape[0]
    y = np.zeros((T, widths[-1]))
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        n = c1 - c0
        a, b, Cm, p, w = gate_coefficients(alpha[c0:c1], eta[c0:c1], beta[c0:c1])
        Q, K, V = q[c0:c1], k[c0:c1], v[c0:c1]
        Hk, Zk = [K], [None]
        for l in range(1, L + 1):
            Z = Hk[l - 1] @ W[l].T
            Zk.append(Z)
            Hk.append(_silu(Z) if l < L else Z)
        D = [None] * (L + 1)
        D[L] = 2.0 * (Zk[L] - V)
        for l in range(L, 1, -1):
            D[l - 1] = (D[l] @ W[l]) * _silu_p(Zk[l - 1])
        Hq = Q
        for l in range(1, L + 1):
            U = (a[:n, None] * (Hq @ W[l].T) - b[:n, None] * (Hq @ S[l].T)
                 - (Cm[:n] * (Hq @ Hk[l - 1].T)) @ D[l])
            Hq = _silu(U) if l < L else U
        y[c0:c1] = Hq
        for l in range(1, L + 1):
            Wn = a[n] * W[l] - b[n] * S[l] - D[l].T @ (Cm[n][:, None] * Hk[l - 1])
            Sn = p * S[l] + D[l].T @ (w[:, None] * Hk[l - 1])
            W[l], S[l] = Wn, Sn
    return y, join(W), join(S)


def chunk_scan(q, k, v, alpha, eta, beta, theta0, s0, C, widths):
    """[B,T,H,d] layout like the oracle; theta0/s0 [H,P] or [B,H,P]."""
    B, T, H, d = q.shape
    P = theta0.shape[-1]
    th0 = np.broadcast_to(theta0, (B, H, P)) if theta0.ndim == 2 else theta0
    sg0 = np.broadcast_to(s0, (B, H, P)) if s0.ndim == 2 else s0
    y = np.zeros((B, T, H, d))
    thT = np.zeros((B, H, P))
    sT = np.zeros((B, H, P))
    for bb in range(B):
        for h in range(H):
            y[bb, :, h], thT[bb, h], sT[bb, h] = chunk_scan_seq(
                q[bb, :, h], k[bb, :, h], v[bb, :, h], alpha[bb, :, h], eta[bb, :, h],
                beta[bb, :, h], th0[bb, h], sg0[bb, h], C, widths)
    return y, thT, sT
