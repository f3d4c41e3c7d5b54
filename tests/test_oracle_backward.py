"""Pins for the oracle's gradients (reverse mode through the token steps).

The gradients are checked against central finite differences of the forward
oracle (a separate code path: the forward never forms an adjoint), component by
component, for L = sum(dy * y) + sum(dS_T * S_T), and against closed forms:
with alpha == 1 and beta == 0 the read-out is y_t = (S_0^T q_t) * sigmoid(z_t),
whose gradients are written out by hand.
"""
import numpy as np
import pytest

import oracle

KEYS = ("q", "k", "v", "log_alpha", "beta", "gate")


def _inputs(rng, B, T, H, Dk, Dv, la_lo=-2.0):
    return dict(q=(rng.standard_normal((B, T, H, Dk)) * 0.5),
                k=(rng.standard_normal((B, T, H, Dk)) * 0.5),
                v=rng.standard_normal((B, T, H, Dv)),
                log_alpha=rng.uniform(la_lo, -0.05, (B, T, H, Dk)),
                beta=rng.uniform(0.1, 0.9, (B, T, H)),
                gate=rng.standard_normal((B, T, H, Dv)))


def _loss(x, s0, dy, dST, clamp=True, **opts):
    y, sT = oracle.fwd(*(x[k].astype(np.float32) for k in KEYS), initial_state=s0, clamp=clamp, **opts)
    return float((y * dy).sum() + (sT * dST).sum())


def _fd(x, s0, dy, dST, name, idx, h=1e-3, clamp=True, **opts):
    """Central difference in float32 input space (the oracle reads fp32): the step is a
    power of two, so x +- h is exact for |x| < 2^13 h and the quotient is (L+ - L-) / 2h."""
    xp = {k: v.astype(np.float32).copy() for k, v in x.items()}
    xm = {k: v.astype(np.float32).copy() for k, v in x.items()}
    xp[name][idx] += np.float32(h)
    xm[name][idx] -= np.float32(h)
    return (_loss(xp, s0, dy, dST, clamp, **opts) - _loss(xm, s0, dy, dST, clamp, **opts)) / (2 * h)


@pytest.mark.parametrize("B,T,H,Dk,Dv", [(1, 1, 1, 2, 3), (1, 5, 2, 3, 2), (2, 4, 1, 4, 4)])
def test_gradients_match_central_differences(oracle_lib, B, T, H, Dk, Dv):
    rng = np.random.default_rng(700 + T * 10 + Dk)
    x = {k: v.astype(np.float32) for k, v in _inputs(rng, B, T, H, Dk, Dv).items()}
    s0 = rng.standard_normal((B, H, Dk, Dv)) * 0.5
    dy = rng.standard_normal((B, T, H, Dv))
    dST = rng.standard_normal((B, H, Dk, Dv))
    g = oracle.bwd(*(x[k] for k in KEYS), dy, initial_state=s0, d_final_state=dST)
    h = 2.0 ** -10
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("log_alpha", "dlog_alpha"),
                        ("beta", "dbeta"), ("gate", "dgate")):
        for idx in np.ndindex(x[name].shape):
            fd = _fd(x, s0, dy, dST, name, idx, h=h)
            an = g[gname][idx]
            # O(h^2) truncation: third derivatives are O(1) here
            assert abs(fd - an) <= 2e-5 * (1 + abs(an)), (name, idx, fd, an)
    # the initial state enters linearly with double precision: difference in double
    for idx in list(np.ndindex(s0.shape))[:12]:
        sp, sm = s0.copy(), s0.copy()
        sp[idx] += 1e-6
        sm[idx] -= 1e-6
        fd = (_loss(x, sp, dy, dST) - _loss(x, sm, dy, dST)) / 2e-6
        assert abs(fd - g["dinitial_state"][idx]) <= 1e-7 * (1 + abs(fd))


def test_clamped_log_alpha_gets_no_gradient(oracle_lib):
    rng = np.random.default_rng(710)
    x = {k: v.astype(np.float32) for k, v in _inputs(rng, 1, 4, 1, 3, 2).items()}
    x["log_alpha"][0, 1, 0, 0] = -9.0  # below the floor
    x["log_alpha"][0, 2, 0, 1] = 0.5   # above retention 1
    dy = rng.standard_normal((1, 4, 1, 2))
    g = oracle.bwd(*(x[k] for k in KEYS), dy)
    assert g["dlog_alpha"][0, 1, 0, 0] == 0.0 and g["dlog_alpha"][0, 2, 0, 1] == 0.0
    # without the clamp the same entries do get a gradient, and it matches a difference
    g2 = oracle.bwd(*(x[k] for k in KEYS), dy, clamp=False)
    z = np.zeros((1, 1, 2, 3))
    for idx in ((0, 1, 0, 0), (0, 2, 0, 1)):
        fd = _fd(x, None, dy, np.zeros((1, 1, 3, 2)), "log_alpha", idx, h=2.0 ** -10, clamp=False)
        assert abs(fd - g2["dlog_alpha"][idx]) <= 2e-5 * (1 + abs(fd))


def test_closed_form_without_writes(oracle_lib):
    """alpha == 1, beta == 0: S_t = S_0, y_t = (S_0^T q_t) * s_t with s_t = sigmoid(z_t).
    Then dq_t = S_0 (dy_t s_t), dS_0 = sum_t q_t (dy_t s_t)^T, dgate_t = dy_t o_t s_t (1 - s_t),
    dv = dk = 0, and dbeta_t = (G_t^T k_t) . (v_t - S_0^T k_t) with G_t = sum_{s >= t} q_s (dy_s s_s)^T."""
    rng = np.random.default_rng(720)
    B, T, H, Dk, Dv = 1, 6, 2, 4, 3
    x = {k: v.astype(np.float32) for k, v in _inputs(rng, B, T, H, Dk, Dv).items()}
    x["log_alpha"][:] = 0.0
    x["beta"][:] = 0.0
    s0 = rng.standard_normal((B, H, Dk, Dv))
    dy = rng.standard_normal((B, T, H, Dv))
    g = oracle.bwd(*(x[k] for k in KEYS), dy, initial_state=s0)
    q, k, v, z = (x[n].astype(np.float64) for n in ("q", "k", "v", "gate"))
    sg = 1 / (1 + np.exp(-z))
    for h in range(H):
        S0 = s0[0, h]
        do = dy[0, :, h] * sg[0, :, h]                      # [T, Dv]
        o = q[0, :, h] @ S0                                 # [T, Dv]
        assert np.allclose(g["dq"][0, :, h], do @ S0.T, rtol=1e-12, atol=1e-13)
        assert np.allclose(g["dinitial_state"][0, h], q[0, :, h].T @ do, rtol=1e-12, atol=1e-13)
        assert np.allclose(g["dgate"][0, :, h], dy[0, :, h] * o * sg[0, :, h] * (1 - sg[0, :, h]),
                           rtol=1e-12, atol=1e-13)
        assert not g["dv"][0, :, h].any() and not g["dk"][0, :, h].any()
        for t in range(T):
            Gt = q[0, t:, h].T @ do[t:]                     # [Dk, Dv]
            want = (Gt.T @ k[0, t, h]) @ (v[0, t, h] - S0.T @ k[0, t, h])
            assert abs(g["dbeta"][0, t, h] - want) <= 1e-12 * (1 + abs(want))


@pytest.mark.parametrize("opts", [dict(qk_norm=True), dict(gate_logits=True), dict(qk_norm=True, gate_logits=True)],
                         ids=["qk_norm", "gate_logits", "both"])
def test_gradients_with_fused_preparation_match_central_differences(oracle_lib, opts):
    """Raw q, k (normalised per token inside, q also by 1/sqrt(Dk)) and forget logits
    (log alpha = logsigmoid(x), then the clamp): the gradients with respect to the raw
    inputs against central differences of the forward oracle given the same raw inputs.
    Logits around -5 put some tokens' retention under the floor, where the clamp stops
    the gradient."""
    rng = np.random.default_rng(740)
    B, T, H, Dk, Dv = 1, 4, 2, 3, 2
    x = {k: v.astype(np.float32) for k, v in _inputs(rng, B, T, H, Dk, Dv).items()}
    x["q"] = (x["q"] * 3.0).astype(np.float32)  # raw projections of any size
    x["k"] = (x["k"] * 0.3).astype(np.float32)
    if opts.get("gate_logits"):
        x["log_alpha"] = rng.uniform(-6.5, 3.0, x["log_alpha"].shape).astype(np.float32)
    s0 = rng.standard_normal((B, H, Dk, Dv)) * 0.5
    dy = rng.standard_normal((B, T, H, Dv))
    dST = rng.standard_normal((B, H, Dk, Dv))
    g = oracle.bwd(*(x[k] for k in KEYS), dy, initial_state=s0, d_final_state=dST, **opts)
    h = 2.0 ** -11
    clamped = 0
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("log_alpha", "dlog_alpha"),
                        ("beta", "dbeta"), ("gate", "dgate")):
        for idx in np.ndindex(x[name].shape):
            xv = float(x[name][idx])
            if name == "log_alpha" and opts.get("gate_logits"):
                ls = min(xv, 0.0) - np.log1p(np.exp(-abs(xv)))
                if abs(ls - oracle.LOG_ALPHA_MIN) < 4 * h:  # the clamp's kink: no difference there
                    continue
                clamped += ls < oracle.LOG_ALPHA_MIN
            fd = _fd(x, s0, dy, dST, name, idx, h=h, **opts)
            an = g[gname][idx]
            assert abs(fd - an) <= 5e-5 * (1 + abs(an)), (name, idx, fd, an)
    if opts.get("gate_logits"):
        assert clamped > 0  # some logits sit under the floor: their gradient is zero
