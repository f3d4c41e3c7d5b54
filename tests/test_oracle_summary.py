"""Pins for the oracle's segment summary and its ordered combination.

Page "3T models are no longer magic", section "KDA context parallelism", and
page "Kimi K3 report walk-through", section "KDA Context Parallelism": a run of
tokens is summarised by how it transforms the incoming state (M) and by the
state it produces from a zero start (b); the segments' summaries are combined in
order to hand each segment its true incoming state.  The checks are the explicit
matrix product, the forward recurrence (a separate code path of the oracle),
the composition law, and closed forms of the delta rule.
"""
import numpy as np
import pytest
import torch

import oracle
from tests._brute import brute_fwd, brute_summary


def _inputs(rng, B, T, H, Dk, Dv, la_lo=-2.0, unit_k=False):
    q = (rng.standard_normal((B, T, H, Dk)) * 0.3).astype(np.float32)
    k = rng.standard_normal((B, T, H, Dk))
    k = k / np.linalg.norm(k, axis=-1, keepdims=True) if unit_k else k * 0.4
    k = k.astype(np.float32)
    v = rng.standard_normal((B, T, H, Dv)).astype(np.float32)
    la = rng.uniform(la_lo, 0.0, (B, T, H, Dk)).astype(np.float32)
    beta = rng.uniform(0.05, 0.95, (B, T, H)).astype(np.float32)
    gate = rng.standard_normal((B, T, H, Dv)).astype(np.float32)
    return q, k, v, la, beta, gate


def _close(a, b, rel=1e-12):
    return np.abs(a - b).max() <= rel * max(np.abs(b).max(), 1e-30)


@pytest.mark.parametrize("B,T,H,Dk,Dv", [(1, 1, 1, 1, 1), (1, 5, 2, 3, 5), (2, 8, 1, 6, 4)])
def test_summary_matches_explicit_matrix_product(oracle_lib, B, T, H, Dk, Dv):
    rng = np.random.default_rng(300 + T + Dk)
    _, k, v, la, beta, _ = _inputs(rng, B, T, H, Dk, Dv, la_lo=-8.0)  # some below the floor
    M, b = oracle.summary(k, v, la, beta)
    Mb, bb = brute_summary(k, v, la, beta)
    assert _close(M, Mb) and _close(b, bb)


def test_summary_bf16_inputs_match_brute_force(oracle_lib):
    rng = np.random.default_rng(301)
    _, k, v, la, beta, _ = _inputs(rng, 1, 7, 2, 5, 3)
    bf = [torch.from_numpy(a).to(torch.bfloat16) for a in (k, v, la, beta)]
    M, b = oracle.summary(*bf)
    Mb, bb = brute_summary(*[t.to(torch.float64).numpy() for t in bf])
    assert _close(M, Mb) and _close(b, bb)


def test_zero_start_state_is_the_forward_final_state(oracle_lib):
    """b is what the forward recurrence reaches from S_0 = 0 (brute force as well)."""
    rng = np.random.default_rng(302)
    x = _inputs(rng, 1, 6, 2, 4, 3)
    _, b = oracle.summary(*(x[i] for i in (1, 2, 3, 4)))
    _, sb = brute_fwd(*x)
    assert _close(b, sb)


def test_forward_is_the_affine_map(oracle_lib):
    """For any S_0, the forward's final state equals M S_0 + b."""
    rng = np.random.default_rng(303)
    q, k, v, la, beta, gate = _inputs(rng, 2, 40, 3, 6, 5)
    M, b = oracle.summary(k, v, la, beta)
    for _ in range(2):
        s0 = rng.standard_normal((2, 3, 6, 5))
        _, sT = oracle.fwd(q, k, v, la, beta, gate, initial_state=s0)
        assert _close(np.matmul(M, s0) + b, sT, 1e-12)


def test_composition_law(oracle_lib):
    """Summary of [0, T) = summary of [T1, T) after [0, T1): M = M2 M1, b = M2 b1 + b2."""
    rng = np.random.default_rng(304)
    _, k, v, la, beta, _ = _inputs(rng, 1, 30, 2, 5, 4)
    M, b = oracle.summary(k, v, la, beta)
    sl = lambda a, lo, hi: np.ascontiguousarray(a[:, lo:hi])
    M1, b1 = oracle.summary(*(sl(a, 0, 11) for a in (k, v, la, beta)))
    M2, b2 = oracle.summary(*(sl(a, 11, 30) for a in (k, v, la, beta)))
    assert _close(np.matmul(M2, M1), M) and _close(np.matmul(M2, b1) + b2, b)


def test_combine_hands_each_segment_its_incoming_state(oracle_lib):
    """combine() of the segments' summaries gives the forward's state at every
    segment boundary, and re-running each segment from it gives the whole output."""
    rng = np.random.default_rng(305)
    B, T, H, Dk, Dv = 1, 37, 2, 6, 4
    x = _inputs(rng, B, T, H, Dk, Dv)
    s0 = rng.standard_normal((B, H, Dk, Dv)) * 0.3
    cuts = [0, 9, 10, 25, 37]
    sl = lambda a, lo, hi: np.ascontiguousarray(a[:, lo:hi])
    sums = [oracle.summary(*(sl(x[i], lo, hi) for i in (1, 2, 3, 4))) for lo, hi in zip(cuts, cuts[1:])]
    seg, fin = oracle.combine(np.stack([m for m, _ in sums]), np.stack([b for _, b in sums]), s0)
    y, sT = oracle.fwd(*x, initial_state=s0)
    assert _close(fin, sT)
    for p, (lo, hi) in enumerate(zip(cuts, cuts[1:])):
        _, s_lo = oracle.fwd(*(sl(a, 0, lo) for a in x), initial_state=s0)
        assert _close(seg[p], s_lo)
        yp, _ = oracle.fwd(*(sl(a, lo, hi) for a in x), initial_state=seg[p])
        assert _close(yp, y[:, lo:hi])


def test_no_write_no_decay_is_identity(oracle_lib):
    """alpha == 1 and beta == 0: every transition is I, so M = I and b = 0 exactly."""
    rng = np.random.default_rng(306)
    _, k, v, la, beta, _ = _inputs(rng, 1, 9, 2, 4, 3)
    la[:] = 0.0
    beta[:] = 0.0
    M, b = oracle.summary(k, v, la, beta)
    assert np.array_equal(M, np.broadcast_to(np.eye(4), M.shape)) and not b.any()


def test_decay_only_is_the_diagonal_product(oracle_lib):
    """beta == 0: M = Diag(exp(sum_t log alpha_t)), b = 0."""
    rng = np.random.default_rng(307)
    _, k, v, la, beta, _ = _inputs(rng, 1, 12, 2, 5, 3, la_lo=-0.4)
    beta[:] = 0.0
    M, b = oracle.summary(k, v, la, beta)
    tot = la.astype(np.float64).sum(axis=1)  # [B, H, Dk]
    for h in range(2):
        assert _close(M[0, h], np.diag(np.exp(tot[0, h])), 1e-13)
    assert not b.any()


def test_last_unit_key_write_is_exact(oracle_lib):
    """Delta rule with unit k_T and beta_T = 1: S_T^T k_T = v_T for any incoming
    state, so k_T^T M = 0 and k_T^T b = v_T (for any decay and any earlier tokens)."""
    rng = np.random.default_rng(308)
    _, k, v, la, beta, _ = _inputs(rng, 1, 10, 3, 4, 4, la_lo=-5.0, unit_k=True)
    had = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1]], dtype=np.float32) / 2
    k[0, -1] = had  # exactly unit length in fp32
    beta[:, -1] = 1.0
    M, b = oracle.summary(k, v, la, beta)
    kT = k[0, -1].astype(np.float64)  # [H, Dk]
    for h in range(3):
        assert np.abs(kT[h] @ M[0, h]).max() <= 1e-15
        assert np.abs(kT[h] @ b[0, h] - v[0, -1, h]).max() <= 1e-13


def test_empty_run(oracle_lib):
    z = lambda *s: np.zeros(s, dtype=np.float32)
    M, b = oracle.summary(z(2, 0, 3, 4), z(2, 0, 3, 5), z(2, 0, 3, 4), z(2, 0, 3))
    assert np.array_equal(M, np.broadcast_to(np.eye(4), (2, 3, 4, 4))) and not b.any()
