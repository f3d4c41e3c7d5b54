"""Independent brute-force expansion of the KDA recurrence for tiny inputs.

Used only to pin the fp64 oracle.  Instead of updating S token by token, it
forms every per-token transition as an explicit d_k x d_k matrix,
    A_s = (I - beta_s k_s k_s^T) Diag(alpha_s),
and evaluates the closed form
    S_t = (A_t ... A_1) S_0 + sum_{s<=t} (A_t ... A_{s+1}) beta_s k_s v_s^T,
    y_t = (S_t^T q_t) * sigmoid(z_t),
with products recomputed from scratch for every (t, s) pair.  Cost is
O(T^2 d_k^3), so keep T <= 8 and d small.
"""
import numpy as np

LOG_ALPHA_MIN = np.log(0.0067)


def brute_fwd(q, k, v, log_alpha, beta, gate, s0=None, clamp=True):
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    la, beta, gate = (np.asarray(a, dtype=np.float64) for a in (log_alpha, beta, gate))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if clamp:
        la = np.clip(la, LOG_ALPHA_MIN, 0.0)
    y = np.zeros((B, T, H, Dv))
    sT = np.zeros((B, H, Dk, Dv))
    eye = np.eye(Dk)
    for b in range(B):
        for h in range(H):
            S0 = np.zeros((Dk, Dv)) if s0 is None else np.asarray(s0, np.float64)[b, h]
            A = [(eye - beta[b, t, h] * np.outer(k[b, t, h], k[b, t, h])) @ np.diag(np.exp(la[b, t, h]))
                 for t in range(T)]

            def prod(hi, lo):  # A_hi ... A_lo (empty product = I), 0-based inclusive
                P = eye.copy()
                for j in range(lo, hi + 1):
                    P = A[j] @ P
                return P

            for t in range(T):
                S = prod(t, 0) @ S0
                for s in range(t + 1):
                    S = S + prod(t, s + 1) @ (beta[b, s, h] * np.outer(k[b, s, h], v[b, s, h]))
                o = S.T @ q[b, t, h]
                y[b, t, h] = o / (1.0 + np.exp(-gate[b, t, h]))
                if t == T - 1:
                    sT[b, h] = S
            if T == 0:
                sT[b, h] = S0
    return y, sT


def brute_summary(k, v, log_alpha, beta, clamp=True):
    """Segment summary by explicit matrices: M = A_T ... A_1 as a product of the
    d_k x d_k transition matrices, and b = sum_s (A_T ... A_{s+1}) beta_s k_s v_s^T
    (the closed form of the state reached from zero), products recomputed per s."""
    k, v = (np.asarray(a, dtype=np.float64) for a in (k, v))
    la, beta = (np.asarray(a, dtype=np.float64) for a in (log_alpha, beta))
    B, T, H, Dk = k.shape
    Dv = v.shape[-1]
    if clamp:
        la = np.clip(la, LOG_ALPHA_MIN, 0.0)
    eye = np.eye(Dk)
    M = np.zeros((B, H, Dk, Dk))
    bs = np.zeros((B, H, Dk, Dv))
    for b in range(B):
        for h in range(H):
            A = [(eye - beta[b, t, h] * np.outer(k[b, t, h], k[b, t, h])) @ np.diag(np.exp(la[b, t, h]))
                 for t in range(T)]

            def prod(lo):  # A_{T-1} ... A_lo, 0-based (empty product = I)
                P = eye.copy()
                for j in range(lo, T):
                    P = A[j] @ P
                return P

            M[b, h] = prod(0)
            for s in range(T):
                bs[b, h] += prod(s + 1) @ (beta[b, s, h] * np.outer(k[b, s, h], v[b, s, h]))
    return M, bs
