"""Pins for the oracle's fused preprocessing options.

Page "3T models are no longer magic", section "FlashKDA": the preparation step
includes Q and K normalisation and the forget-gate computation.  The inputs the
kernel is specified on are L2-normalised q and k with q scaled by 1/sqrt(d_k),
and log alpha = max(logsigmoid(x), ln 0.0067) from a logit x (the retention
floor of section "Gate 1: KDA makes it computable").  With ``qk_norm`` and
``gate_logits`` the oracle takes the raw q, k and x and does these steps itself.

Checks: the independent brute force on inputs prepared with numpy/scipy
(``np.linalg.norm``, ``scipy.special.log_expit``), scale invariance, the
delta-rule retrieval on raw keys (which also fixes the 1/sqrt(d_k) query scale),
and the half-retention closed form at x = 0.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import log_expit

import oracle
from tests._brute import LOG_ALPHA_MIN, brute_fwd, brute_summary


def _raw(rng, B, T, H, Dk, Dv):
    # raw projections of very different sizes per token
    q = (rng.standard_normal((B, T, H, Dk)) * rng.uniform(0.05, 20, (B, T, H, 1))).astype(np.float32)
    k = (rng.standard_normal((B, T, H, Dk)) * rng.uniform(0.05, 20, (B, T, H, 1))).astype(np.float32)
    v = rng.standard_normal((B, T, H, Dv)).astype(np.float32)
    x = (rng.standard_normal((B, T, H, Dk)) * 3 + 1).astype(np.float32)  # forget logits, some far below the floor
    beta = rng.uniform(0.05, 0.95, (B, T, H)).astype(np.float32)
    gate = rng.standard_normal((B, T, H, Dv)).astype(np.float32)
    return q, k, v, x, beta, gate


def _prepared(q, k, x):
    q64, k64 = q.astype(np.float64), k.astype(np.float64)
    Dk = q.shape[-1]
    qn = q64 / np.linalg.norm(q64, axis=-1, keepdims=True) / math.sqrt(Dk)
    kn = k64 / np.linalg.norm(k64, axis=-1, keepdims=True)
    la = np.maximum(log_expit(x.astype(np.float64)), LOG_ALPHA_MIN)
    return qn, kn, la


def _close(a, b, rel=1e-12):
    return np.abs(a - b).max() <= rel * max(np.abs(b).max(), 1e-30)


@pytest.mark.parametrize("B,T,H,Dk,Dv", [(1, 6, 2, 5, 3), (2, 8, 1, 4, 4), (1, 1, 3, 7, 2)])
def test_fused_prep_matches_brute_force_on_prepared_inputs(oracle_lib, B, T, H, Dk, Dv):
    rng = np.random.default_rng(500 + T + Dk)
    q, k, v, x, beta, gate = _raw(rng, B, T, H, Dk, Dv)
    s0 = rng.standard_normal((B, H, Dk, Dv)) * 0.3
    y, sT = oracle.fwd(q, k, v, x, beta, gate, initial_state=s0, qk_norm=True, gate_logits=True)
    qn, kn, la = _prepared(q, k, x)
    yb, sb = brute_fwd(qn, kn, v, la, beta, gate, s0=s0, clamp=False)
    assert _close(y, yb) and _close(sT, sb)


def test_each_option_alone(oracle_lib):
    rng = np.random.default_rng(501)
    q, k, v, x, beta, gate = _raw(rng, 1, 7, 2, 4, 3)
    qn, kn, la = _prepared(q, k, x)
    la_plain = np.clip(x, -1.5, 0.0).astype(np.float32)  # already a log alpha
    y, sT = oracle.fwd(q, k, v, la_plain, beta, gate, qk_norm=True)
    yb, sb = brute_fwd(qn, kn, v, la_plain, beta, gate)
    assert _close(y, yb) and _close(sT, sb)
    qs = (q / np.linalg.norm(q, axis=-1, keepdims=True) / 2).astype(np.float32)  # any q, k as given
    y, sT = oracle.fwd(qs, qs, v, x, beta, gate, gate_logits=True)
    yb, sb = brute_fwd(qs, qs, v, la, beta, gate, clamp=False)
    assert _close(y, yb) and _close(sT, sb)


def test_normalisation_is_scale_invariant(oracle_lib):
    """Multiplying a token's raw q or k by a power of two changes nothing."""
    rng = np.random.default_rng(502)
    q, k, v, x, beta, gate = _raw(rng, 1, 9, 2, 6, 4)
    y, sT = oracle.fwd(q, k, v, x, beta, gate, qk_norm=True, gate_logits=True)
    f = (2.0 ** rng.integers(-6, 7, (1, 9, 2, 1))).astype(np.float32)
    y2, s2 = oracle.fwd(q * f, k * f[:, ::-1], v, x, beta, gate, qk_norm=True, gate_logits=True)
    assert _close(y2, y, 1e-13) and _close(s2, sT, 1e-13)


def test_retrieval_with_raw_key_fixes_query_scale(oracle_lib):
    """beta = 1: the normalised key retrieves v exactly; with q equal to the raw key the
    read is v / sqrt(d_k), and a large gate logit passes it through."""
    rng = np.random.default_rng(503)
    B, T, H, Dk, Dv = 1, 5, 2, 16, 3
    q, k, v, x, beta, gate = _raw(rng, B, T, H, Dk, Dv)
    k[..., :] = 0.0
    k[..., 3] = rng.uniform(0.1, 9, (B, T, H)).astype(np.float32)  # raw key: a multiple of e_3
    q = k.copy()
    beta[:] = 1.0
    gate[:] = 40.0
    s0 = rng.standard_normal((B, H, Dk, Dv))
    y, _ = oracle.fwd(q, k, v, x, beta, gate, initial_state=s0, qk_norm=True, gate_logits=True)
    assert np.abs(y - v / math.sqrt(Dk)).max() <= 1e-12 * np.abs(v).max()


def test_zero_logit_halves_retention(oracle_lib):
    """x = 0: alpha = sigmoid(0) = 1/2 exactly; with no writes the summary is 2^-T I."""
    rng = np.random.default_rng(504)
    q, k, v, x, beta, gate = _raw(rng, 1, 6, 2, 4, 3)
    x[:] = 0.0
    beta[:] = 0.0
    M, b = oracle.summary(k, v, x, beta, qk_norm=True, gate_logits=True)
    assert np.abs(M - np.broadcast_to(np.eye(4) / 64.0, M.shape)).max() <= 1e-15 and not b.any()


def test_decode_and_summary_take_the_same_options(oracle_lib):
    rng = np.random.default_rng(505)
    q, k, v, x, beta, gate = _raw(rng, 2, 6, 3, 5, 4)
    s0 = rng.standard_normal((2, 3, 5, 4))
    opts = dict(qk_norm=True, gate_logits=True)
    y, sT = oracle.fwd(q, k, v, x, beta, gate, initial_state=s0, **opts)
    s = s0.copy()
    for t in range(6):
        yt, s = oracle.decode(*(np.ascontiguousarray(a[:, t]) for a in (q, k, v, x, beta, gate)), s, **opts)
        assert _close(yt, y[:, t])
    assert _close(s, sT)
    M, b = oracle.summary(k, v, x, beta, **opts)
    qn, kn, la = _prepared(q, k, x)
    Mb, bb = brute_summary(kn, v, la, beta, clamp=False)
    assert _close(M, Mb) and _close(b, bb)


def test_bf16_raw_inputs(oracle_lib):
    rng = np.random.default_rng(506)
    arrs = _raw(rng, 1, 5, 2, 6, 3)
    bf = [torch.from_numpy(a).to(torch.bfloat16) for a in arrs]
    y, sT = oracle.fwd(*bf, qk_norm=True, gate_logits=True)
    w = [t.to(torch.float64).numpy() for t in bf]
    qn, kn, la = _prepared(*(w[i].astype(np.float32) for i in (0, 1, 3)))  # bf16 values are exact in fp32
    yb, sb = brute_fwd(qn, kn, w[2], la, w[4], w[5], clamp=False)
    assert _close(y, yb) and _close(sT, sb)
