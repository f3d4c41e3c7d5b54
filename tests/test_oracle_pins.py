"""Pins for the fp64 oracle: checks against facts fixed by the pages and by the
mathematics, never against the oracle's own formula retyped.

Pages: "3T models are no longer magic" (p1), section "Gate 1: KDA makes it
computable" (token flow, channel-wise forget, 0.67 % floor, delta rule, output
gate); "Kimi K3 report walk-through" (p2), sections "Compute paradigm" and
"Hierarchical chunking of linear attention" (chunk size does not change the
result) and "Numerical stability & co-design" (16-token tile inside the BF16
range); p1 section "KDA context parallelism" (a segment is summarised by how it
transforms the incoming state plus the state it produces from zero).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests._brute import brute_fwd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_inputs(rng, B, T, H, Dk, Dv, la_lo=-3.0, unit_k=False):
    q = rng.standard_normal((B, T, H, Dk)).astype(np.float32) * 0.3
    k = rng.standard_normal((B, T, H, Dk)).astype(np.float32)
    if unit_k:
        k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    else:
        k = k * 0.4
    k = k.astype(np.float32)
    v = rng.standard_normal((B, T, H, Dv)).astype(np.float32)
    la = rng.uniform(la_lo, 0.0, (B, T, H, Dk)).astype(np.float32)
    beta = rng.uniform(0.05, 0.95, (B, T, H)).astype(np.float32)
    gate = rng.standard_normal((B, T, H, Dv)).astype(np.float32)
    return q, k, v, la, beta, gate


def _hadamard(n):
    Hm = np.array([[1.0]])
    while Hm.shape[0] < n:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    return Hm


# ---------------------------------------------------------------- I3: brute force
@pytest.mark.parametrize("B,T,H,Dk,Dv", [(1, 1, 1, 1, 1), (1, 5, 2, 3, 5), (2, 8, 1, 6, 4),
                                         (1, 7, 3, 4, 4)])
def test_oracle_matches_brute_force_expansion(oracle_lib, B, T, H, Dk, Dv):
    rng = np.random.default_rng(100 + T * 7 + Dk)
    q, k, v, la, beta, gate = _rand_inputs(rng, B, T, H, Dk, Dv)
    s0 = rng.standard_normal((B, H, Dk, Dv)) * 0.5
    y, sT = oracle.fwd(q, k, v, la, beta, gate, initial_state=s0)
    yb, sb = brute_fwd(q, k, v, la, beta, gate, s0=s0)
    scale = max(np.abs(yb).max(), 1e-30)
    assert np.abs(y - yb).max() <= 1e-12 * scale
    assert np.abs(sT - sb).max() <= 1e-12 * max(np.abs(sb).max(), 1e-30)


def test_oracle_matches_brute_force_bf16_inputs(oracle_lib):
    """The oracle widens the exact bf16 bit patterns; brute force on the same values."""
    rng = np.random.default_rng(7)
    arrs = _rand_inputs(rng, 1, 6, 2, 5, 3)
    bf = [torch.from_numpy(a).to(torch.bfloat16) for a in arrs]
    y, sT = oracle.fwd(*bf)
    yb, sb = brute_fwd(*[t.to(torch.float64).numpy() for t in bf])
    assert np.abs(y - yb).max() <= 1e-12 * np.abs(yb).max()
    assert np.abs(sT - sb).max() <= 1e-12 * np.abs(sb).max()


# ------------------------------------------------------------- I1: linear attention
def test_alpha_one_beta_zero_keeps_initial_state(oracle_lib):
    """I1a: alpha == 1 and beta == 0 switch the write off: S_t = S_0, o_t = S_0^T q_t."""
    rng = np.random.default_rng(1)
    B, T, H, Dk, Dv = 1, 9, 2, 4, 6
    q, k, v, la, beta, gate = _rand_inputs(rng, B, T, H, Dk, Dv)
    la[:] = 0.0
    beta[:] = 0.0
    s0 = rng.standard_normal((B, H, Dk, Dv))
    y, sT = oracle.fwd(q, k, v, la, beta, gate, initial_state=s0)
    assert np.array_equal(sT, s0)
    o = np.einsum("bthc,bhcj->bthj", q.astype(np.float64), s0)
    ref = o / (1.0 + np.exp(-gate.astype(np.float64)))
    assert np.abs(y - ref).max() <= 1e-14 * np.abs(ref).max()


@pytest.mark.parametrize("dense", [False, True])
def test_orthogonal_keys_give_causal_linear_attention(oracle_lib, dense):
    """I1b: alpha == 1, orthonormal keys, S_0 = 0: the delta correction reads zero and
    the layer is textbook causal linear attention (mask . Q K^T diag(beta)) V, gated."""
    rng = np.random.default_rng(2)
    Dk, Dv, T = 16, 5, 12
    if dense:  # rows of a Sylvester Hadamard matrix / 4 are exactly orthonormal in fp32
        basis = _hadamard(Dk) / 4.0
    else:
        basis = np.eye(Dk)
    rows = rng.permutation(Dk)[:T]
    k = basis[rows].astype(np.float32)[None, :, None, :]
    q = (rng.standard_normal((1, T, 1, Dk)) * 0.5).astype(np.float32)
    v = rng.standard_normal((1, T, 1, Dv)).astype(np.float32)
    la = np.zeros((1, T, 1, Dk), np.float32)
    beta = rng.uniform(0.1, 0.9, (1, T, 1)).astype(np.float32)
    gate = rng.standard_normal((1, T, 1, Dv)).astype(np.float32)
    y, sT = oracle.fwd(q, k, v, la, beta, gate)
    Q, K, V = (a[0, :, 0].astype(np.float64) for a in (q, k, v))
    Bt = beta[0, :, 0].astype(np.float64)
    attn = np.tril(Q @ K.T) * Bt[None, :]
    ref = (attn @ V) / (1.0 + np.exp(-gate[0, :, 0].astype(np.float64)))
    assert np.abs(y[0, :, 0] - ref).max() <= 1e-13 * np.abs(ref).max()
    assert np.abs(sT[0, 0] - (K.T * Bt) @ V).max() <= 1e-13


def test_first_order_in_beta_is_linear_attention(oracle_lib):
    """I1c: with alpha == 1 and S_0 = 0, dS_T/dbeta at beta = 0 (all tokens) is
    sum_s k_s v_s^T; central differences with an exactly representable step."""
    rng = np.random.default_rng(3)
    B, T, H, Dk, Dv = 1, 10, 1, 6, 4
    q, k, v, la, beta, gate = _rand_inputs(rng, B, T, H, Dk, Dv)
    la[:] = 0.0
    eps = np.float32(2.0 ** -20)
    _, sp = oracle.fwd(q, k, v, la, np.full_like(beta, eps), gate)
    _, sm = oracle.fwd(q, k, v, la, np.full_like(beta, -eps), gate)
    fd = (sp - sm) / (2.0 * float(eps))
    ref = np.einsum("tc,tj->cj", k[0, :, 0].astype(np.float64), v[0, :, 0].astype(np.float64))
    assert np.abs(fd[0, 0] - ref).max() <= 1e-9 * np.abs(ref).max()


# ----------------------------------------------------------------- I2: delta rule
def test_delta_rule_exact_retrieval(oracle_lib):
    """I2: with unit-norm k_t and beta_t = 1, the written state returns v_t when read
    with k_t, for any decay and any prior state ((I - k k^T) k = 0).  Reading with
    q_t = k_t and gate logit 0 therefore gives y_t = v_t / 2 at every token."""
    rng = np.random.default_rng(4)
    Dk, Dv, T = 64, 7, 20
    signs = rng.choice([-1.0, 1.0], size=(1, T, 1, Dk))
    k = (signs / 8.0).astype(np.float32)  # entries +-1/8: norm exactly 1 for d_k = 64
    v = rng.standard_normal((1, T, 1, Dv)).astype(np.float32)
    la = rng.uniform(-5.0, 0.0, (1, T, 1, Dk)).astype(np.float32)
    beta = np.ones((1, T, 1), np.float32)
    gate = np.zeros((1, T, 1, Dv), np.float32)
    s0 = rng.standard_normal((1, 1, Dk, Dv))
    y, sT = oracle.fwd(k.copy(), k, v, la, beta, gate, initial_state=s0)
    assert np.abs(y - v.astype(np.float64) / 2.0).max() <= 1e-12
    assert np.abs(sT[0, 0].T @ k[0, -1, 0].astype(np.float64) - v[0, -1, 0]).max() <= 1e-12


def test_rewriting_same_pair_is_idempotent(oracle_lib):
    """I2b: I - k k^T is a projector, so writing (k, v) twice with beta = 1, alpha = 1
    leaves the state of the first write unchanged."""
    rng = np.random.default_rng(5)
    Dk, Dv = 64, 3
    kk = (rng.choice([-1.0, 1.0], size=Dk) / 8.0).astype(np.float32)
    vv = rng.standard_normal(Dv).astype(np.float32)
    k = np.stack([kk, kk])[None, :, None, :]
    v = np.stack([vv, vv])[None, :, None, :]
    q = np.zeros_like(k)
    la = np.zeros_like(k)
    beta = np.ones((1, 2, 1), np.float32)
    gate = np.zeros((1, 2, 1, Dv), np.float32)
    s0 = rng.standard_normal((1, 1, Dk, Dv))
    _, s1 = oracle.fwd(q[:, :1], k[:, :1], v[:, :1], la[:, :1], beta[:, :1], gate[:, :1],
                       initial_state=s0)
    _, s2 = oracle.fwd(q, k, v, la, beta, gate, initial_state=s0)
    assert np.abs(s2 - s1).max() <= 1e-13


# ---------------------------------------------------------------------- I4: gate
def test_gate_closed_forms(oracle_lib):
    """I4: z = 0 halves the read-out exactly; z = 40 passes it through."""
    rng = np.random.default_rng(6)
    q, k, v, la, beta, gate = _rand_inputs(rng, 1, 6, 2, 5, 4)
    y0, _ = oracle.fwd(q, k, v, la, beta, np.zeros_like(gate))
    y1, _ = oracle.fwd(q, k, v, la, beta, np.full_like(gate, 40.0))
    assert np.abs(y1 - 2.0 * y0).max() <= 1e-14 * np.abs(y1).max()
    yb, _ = brute_fwd(q, k, v, la, beta, np.full_like(gate, 40.0))
    assert np.abs(y1 - yb).max() <= 1e-12 * np.abs(yb).max()


# ------------------------------------------------------- floor / clamp (O1, O2)
def test_clamp_to_retention_floor(oracle_lib):
    """log alpha below ln 0.0067 acts as the floor, above 0 acts as 0; without the
    clamp the raw value is used (checked against the brute force both ways)."""
    rng = np.random.default_rng(8)
    q, k, v, la, beta, gate = _rand_inputs(rng, 1, 7, 1, 4, 3)
    la = rng.uniform(-12.0, 2.0, la.shape).astype(np.float32)
    y, sT = oracle.fwd(q, k, v, la, beta, gate, clamp=True)
    yb, sb = brute_fwd(q, k, v, np.clip(la.astype(np.float64), math.log(0.0067), 0.0), beta, gate,
                      clamp=False)
    assert np.abs(y - yb).max() <= 1e-12 * np.abs(yb).max()
    y2, _ = oracle.fwd(q, k, v, la, beta, gate, clamp=False)
    yb2, _ = brute_fwd(q, k, v, la, beta, gate, clamp=False)
    assert np.abs(y2 - yb2).max() <= 1e-12 * np.abs(yb2).max()
    assert np.abs(y2 - y).max() > 1e-6  # the clamp is not a no-op on these inputs


# --------------------------------------------- I6: chunk/segment split, affinity
def test_split_and_chain_equals_whole(oracle_lib):
    """Running [0, T1) then [T1, T) from the chained state equals one run over [0, T)
    (the segment handoff of KDA context parallelism; chunk size does not matter)."""
    rng = np.random.default_rng(9)
    q, k, v, la, beta, gate = _rand_inputs(rng, 2, 40, 3, 8, 6, unit_k=True)
    s0 = rng.standard_normal((2, 3, 8, 6)) * 0.1
    y, sT = oracle.fwd(q, k, v, la, beta, gate, initial_state=s0)
    for T1 in (1, 16, 23, 39):
        sl = lambda a, lo, hi: np.ascontiguousarray(a[:, lo:hi])
        ya, sa = oracle.fwd(*(sl(a, 0, T1) for a in (q, k, v, la, beta, gate)), initial_state=s0)
        yb, sb = oracle.fwd(*(sl(a, T1, 40) for a in (q, k, v, la, beta, gate)), initial_state=sa)
        assert np.abs(np.concatenate([ya, yb], axis=1) - y).max() <= 1e-13
        assert np.abs(sb - sT).max() <= 1e-13


def test_output_is_affine_in_initial_state(oracle_lib):
    """S_T and y are affine in S_0 (a segment = a linear map plus a zero-start state)."""
    rng = np.random.default_rng(10)
    q, k, v, la, beta, gate = _rand_inputs(rng, 1, 30, 2, 6, 5, unit_k=True)
    sa = rng.standard_normal((1, 2, 6, 5))
    sb = rng.standard_normal((1, 2, 6, 5))
    y0, s0 = oracle.fwd(q, k, v, la, beta, gate)
    ya, s_a = oracle.fwd(q, k, v, la, beta, gate, initial_state=sa)
    yb, s_b = oracle.fwd(q, k, v, la, beta, gate, initial_state=sb)
    yab, s_ab = oracle.fwd(q, k, v, la, beta, gate, initial_state=sa + 2.0 * sb)
    assert np.abs((yab - y0) - ((ya - y0) + 2.0 * (yb - y0))).max() <= 1e-12
    assert np.abs((s_ab - s0) - ((s_a - s0) + 2.0 * (s_b - s0))).max() <= 1e-12


# ---------------------------------------------------------------- I7: padding
def test_identity_tokens_change_nothing(oracle_lib):
    """Appending tokens with beta = 0, log alpha = 0 and k = 0 leaves the state and the
    earlier outputs unchanged: (I - 0) I S + 0 = S."""
    rng = np.random.default_rng(11)
    q, k, v, la, beta, gate = _rand_inputs(rng, 1, 13, 2, 5, 4)
    y, sT = oracle.fwd(q, k, v, la, beta, gate)
    pad = 7
    cat = lambda a, fill: np.concatenate([a, fill], axis=1)
    qp = cat(q, rng.standard_normal((1, pad, 2, 5)).astype(np.float32))
    kp = cat(k, np.zeros((1, pad, 2, 5), np.float32))
    vp = cat(v, rng.standard_normal((1, pad, 2, 4)).astype(np.float32))
    lap = cat(la, np.zeros((1, pad, 2, 5), np.float32))
    bp = cat(beta, np.zeros((1, pad, 2), np.float32))
    gp = cat(gate, rng.standard_normal((1, pad, 2, 4)).astype(np.float32))
    y2, s2 = oracle.fwd(qp, kp, vp, lap, bp, gp)
    assert np.array_equal(s2, sT)
    assert np.array_equal(y2[:, :13], y)


def test_empty_sequence(oracle_lib):
    rng = np.random.default_rng(12)
    q, k, v, la, beta, gate = _rand_inputs(rng, 2, 0, 3, 4, 4)
    s0 = rng.standard_normal((2, 3, 4, 4))
    y, sT = oracle.fwd(q, k, v, la, beta, gate, initial_state=s0)
    assert y.shape == (2, 0, 3, 4)
    assert np.array_equal(sT, s0)
    _, z = oracle.fwd(q, k, v, la, beta, gate)
    assert not z.any()


# -------------------------------------------------------- I8: decode vs prefill
def test_decode_steps_equal_prefill(oracle_lib):
    rng = np.random.default_rng(13)
    q, k, v, la, beta, gate = _rand_inputs(rng, 2, 6, 3, 5, 4)
    s0 = rng.standard_normal((2, 3, 5, 4))
    y, sT = oracle.fwd(q, k, v, la, beta, gate, initial_state=s0)
    s = s0
    for t in range(6):
        yt, s = oracle.decode(*(np.ascontiguousarray(a[:, t]) for a in (q, k, v, la, beta, gate)), s)
        assert np.abs(yt - y[:, t]).max() <= 1e-14
    assert np.abs(s - sT).max() <= 1e-14


# ---------------------------------------------- I10: the pages' BF16-range claim
def test_sixteen_token_tile_fits_bf16_range():
    """p2 "Numerical stability & co-design": the largest decay inside a 16-token tile,
    derived backwards from the BF16 range, must stay representable.  With the p1
    floor (about 0.67 % retention), 16 steps give e^80.1 < bf16 max, 17 still fit,
    18 overflow; so 16 is the largest power-of-two tile."""
    with open(os.path.join(GOLDEN, "page_constants.json")) as f:
        c = json.load(f)
    floor = c["retention_floor"]["value"]
    tile = c["bf16_tile_tokens"]["value"]
    bf16_max = float(torch.finfo(torch.bfloat16).max)
    bf16_tiny = float(torch.finfo(torch.bfloat16).tiny)
    assert abs(bf16_max - c["bf16_max"]["value"]) / bf16_max < 0.01
    per_step = -math.log(floor)
    assert tile * per_step < math.log(bf16_max)
    assert -tile * per_step > math.log(bf16_tiny)
    assert 17 * per_step < math.log(bf16_max) < 18 * per_step
    # the floor in bf16 is exactly -5.0, inside [ln 0.0067, 0]
    f_bf16 = torch.tensor(math.log(floor)).to(torch.bfloat16).item()
    assert f_bf16 == -5.0 and f_bf16 >= math.log(floor)
    # half of a tile (the reference point used for 16-token pair products) is ~e^40
    assert math.exp(8 * per_step) < 3e17
