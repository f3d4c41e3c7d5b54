"""The chunkwise form of KDA and its adjoint, in fp64 numpy, chunk by chunk.

Forward of one chunk from the state S0 at its start (tokens r, s = 1..C; g the
inclusive cumulative log-decay, G = e^g per row and channel; Gc = e^{g_C}):
    Kt = K G,  Qt = Q G,  Ki = K / G,  Kb = K (Gc / G)
    A = strict_lower(diag(beta) Kt Ki^T),  P = lower(Qt Ki^T),  L = I + A
    U = L^-1 diag(beta) (V - Kt S0)
    O = Qt S0 + P U,   S_C = Diag(Gc) S0 + Kb^T U,   Y = O * sigmoid(Z)
The adjoint takes dY and dS_C back through these steps to dQ, dK, dV, dbeta,
dlog alpha (a reverse cumulative sum of dg), dZ and dS0.  Everything is formed
relative to the chunk start, so e^{-g} may be large: fine in fp64 for the small
cases this is used on.  This is the algebra a chunkwise backward follows; it is
checked against the oracle's token-by-token gradients.
"""
import numpy as np

LOG_ALPHA_MIN = np.log(0.0067)


def _chunk(q, k, v, lam, beta, z, S0):
    g = np.cumsum(lam, axis=0)
    G, Gc = np.exp(g), np.exp(g[-1])
    Kt, Qt, Ki, Kb = k * G, q * G, k / G, k * (Gc / G)
    C = q.shape[0]
    A = np.tril(beta[:, None] * (Kt @ Ki.T), -1)
    P = np.tril(Qt @ Ki.T)
    L = np.eye(C) + A
    Linv = np.linalg.inv(L)
    X = v - Kt @ S0
    U = Linv @ (beta[:, None] * X)
    O = Qt @ S0 + P @ U
    SC = Gc[:, None] * S0 + Kb.T @ U
    sg = 1 / (1 + np.exp(-z))
    return dict(g=g, G=G, Gc=Gc, Kt=Kt, Qt=Qt, Ki=Ki, Kb=Kb, A=A, P=P, Linv=Linv, X=X, U=U, O=O,
                SC=SC, sg=sg, Y=O * sg)


def _chunk_adjoint(f, q, k, v, beta, S0, dY, dSC):
    C = q.shape[0]
    sg = f["sg"]
    dZ = dY * f["O"] * sg * (1 - sg)
    dO = dY * sg
    # O = Qt S0 + P U
    dQt = dO @ S0.T
    dS0 = f["Qt"].T @ dO
    dP = np.tril(dO @ f["U"].T)
    dU = f["P"].T @ dO
    # S_C = Diag(Gc) S0 + Kb^T U
    dGc = (dSC * S0).sum(axis=1)
    dS0 += f["Gc"][:, None] * dSC
    dKb = f["U"] @ dSC.T
    dU += f["Kb"] @ dSC
    # U = Linv diag(beta) X
    Linv = f["Linv"]
    W = beta[:, None] * f["X"]
    dLinv = dU @ W.T
    dW = Linv.T @ dU
    dbeta = (dW * f["X"]).sum(axis=1)
    dX = beta[:, None] * dW
    dV = dX
    dKt = -dX @ S0.T
    dS0 += -f["Kt"].T @ dX
    # Linv = L^-1: dL = -L^-T dLinv L^-T;  A = strict_lower(diag(beta) Kt Ki^T)
    dA = np.tril(-Linv.T @ dLinv @ Linv.T, -1)
    B = np.tril(f["Kt"] @ f["Ki"].T, -1)
    dbeta += (dA * B).sum(axis=1)
    dKt += (beta[:, None] * dA) @ f["Ki"]
    dKi = (beta[:, None] * dA).T @ f["Kt"]
    # P = lower(Qt Ki^T)
    dQt += dP @ f["Ki"]
    dKi += dP.T @ f["Qt"]
    # back to q, k and g
    G, Gc = f["G"], f["Gc"]
    dq = dQt * G
    dk = dKt * G + dKi / G + dKb * (Gc / G)
    dg = dQt * f["Qt"] + dKt * f["Kt"] - dKi * f["Ki"] - dKb * f["Kb"]
    dgC = (dKb * f["Kb"]).sum(axis=0) + dGc * Gc
    dg[-1] += dgC
    dlam = np.cumsum(dg[::-1], axis=0)[::-1]  # g_r = sum_{s <= r} lam_s
    return dict(dq=dq, dk=dk, dv=dV, dbeta=dbeta, dlam=dlam, dz=dZ, dS0=dS0)


def chunkwise_fwd_bwd(q, k, v, log_alpha, beta, gate, dy, s0, dST, chunk, clamp=True):
    """One (b, h) sequence [T, D]: the chunkwise forward (outputs, final state) and the
    chunkwise adjoint (gradients), chunks of `chunk` tokens (a last partial chunk is
    simply shorter)."""
    q, k, v, la, beta, gate, dy = (np.asarray(a, np.float64) for a in (q, k, v, log_alpha, beta, gate, dy))
    lam = np.clip(la, LOG_ALPHA_MIN, 0.0) if clamp else la
    T = q.shape[0]
    bounds = [(i, min(i + chunk, T)) for i in range(0, T, chunk)]
    S = np.array(s0, np.float64)
    starts, fwd, y = [], [], np.zeros((T, v.shape[1]))
    for lo, hi in bounds:
        starts.append(S)
        f = _chunk(q[lo:hi], k[lo:hi], v[lo:hi], lam[lo:hi], beta[lo:hi], gate[lo:hi], S)
        fwd.append(f)
        y[lo:hi] = f["Y"]
        S = f["SC"]
    out = {n: np.zeros_like(a) for n, a in (("dq", q), ("dk", k), ("dv", v), ("dlog_alpha", la), ("dgate", gate))}
    out["dbeta"] = np.zeros_like(beta)
    dS = np.array(dST, np.float64)
    for (lo, hi), f, S0 in reversed(list(zip(bounds, fwd, starts))):
        gr = _chunk_adjoint(f, q[lo:hi], k[lo:hi], v[lo:hi], beta[lo:hi], S0, dy[lo:hi], dS)
        out["dq"][lo:hi], out["dk"][lo:hi], out["dv"][lo:hi] = gr["dq"], gr["dk"], gr["dv"]
        out["dbeta"][lo:hi], out["dgate"][lo:hi] = gr["dbeta"], gr["dz"]
        out["dlog_alpha"][lo:hi] = gr["dlam"]
        dS = gr["dS0"]
    if clamp:
        out["dlog_alpha"] *= (la >= LOG_ALPHA_MIN) & (la <= 0.0)
    out["dinitial_state"] = dS
    return y, S, out
