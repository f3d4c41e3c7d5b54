"""GPU parity of the segment summary and the ordered combination (through the C
ABI) against the fp64 oracle.

Page "3T models are no longer magic", section "KDA context parallelism", and page
"Kimi K3 report walk-through", section "KDA Context Parallelism": a run of tokens
maps the state it receives to M S + b; summaries of consecutive runs combine in
order into each run's incoming state, from which the run is re-computed.

Error measures (max |gpu - oracle| over the tensor):
  b, states, outputs: / rms(oracle), as for kda_chunk_fwd: 2e-2 (bf16 inputs),
    1e-4 (fp32 inputs of the combination);
  M: / max(rms(M_oracle), 1/sqrt(d_k)).  The recurrence is non-expansive, so the
    identity map is the largest transition a run can have; over long runs with
    strong decay, or many delta-rule writes, M itself shrinks towards zero
    (e^-50 after 300 tokens of the common recipe) and is judged on the
    identity's scale.  Where M is within 10x of that scale (slow decay, weak
    writes), plain err/rms is checked as well.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from kda_workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

TOL_BF16, TOL_F32 = 2e-2, 1e-4
KEYS = ("q", "k", "v", "log_alpha", "beta", "gate")


def kda():
    import gated_delta_rule_106_amd as m
    return m


def say(*a):
    print(*a, flush=True)


def _np(x):
    return x.detach().double().cpu().numpy() if isinstance(x, torch.Tensor) else np.asarray(x, np.float64)


def rel_err(got, ref, floor=0.0):
    got, ref = _np(got), _np(ref)
    if ref.size == 0:
        return 0.0
    rms = math.sqrt(float((ref ** 2).mean()))
    return float(np.abs(got - ref).max()) / max(rms, floor, 1e-30)


def _summary_gpu(x):
    d = {k: x[k].cuda() for k in ("k", "v", "log_alpha", "beta")}
    M, b = kda().chunk_summary(d["k"], d["v"], d["log_alpha"], d["beta"])
    torch.cuda.synchronize()
    return M, b


@pytest.mark.parametrize("B,H,T,D,alpha_mu,beta_mu", [
    (1, 2, 300, 128, 2.0, 0.0), (1, 2, 300, 128, 6.0, 0.0), (2, 1, 64, 64, 2.0, 0.0),
    (1, 3, 1, 128, 2.0, 0.0), (1, 2, 1000, 64, 6.0, 0.0), (1, 4, 4096, 128, 2.0, 0.0),
    (1, 2, 4033, 128, 7.0, 0.0), (1, 2, 700, 128, 7.0, -3.0), (1, 2, 190, 64, 6.0, -3.0)])
def test_summary_matches_oracle(B, H, T, D, alpha_mu, beta_mu):
    wl = CONFIGS[1].scaled(B=B, H=H, T=T, Dk=D, Dv=D, alpha_mu=alpha_mu, beta_mu=beta_mu,
                           init_state=True)
    x = make_inputs(wl, seed=40 + T)
    say(f"[summary] B={B} H={H} T={T} D={D} alpha_mu={alpha_mu} beta_mu={beta_mu}")
    M, b = _summary_gpu(x)
    Mo, bo = oracle.summary(x["k"], x["v"], x["log_alpha"], x["beta"])
    eM = rel_err(M, Mo, floor=1 / math.sqrt(D))
    eb = rel_err(b, bo)
    # the map in use: M S_0 + b against the oracle's forward from a random S_0
    s0 = x["initial_state"].double().numpy() * 50  # N(0, 1) entries: M's share is not negligible
    _, so = oracle.fwd(*(x[k] for k in KEYS), initial_state=s0)
    eS = rel_err(np.matmul(_np(M), s0) + _np(b), so)
    say(f"[summary] M err={eM:.3e} (rms M {math.sqrt(float((Mo ** 2).mean())):.2e}) b err/rms={eb:.3e} "
        f"M S0 + b err/rms={eS:.3e}")
    assert np.isfinite(eM) and eM <= TOL_BF16
    assert np.isfinite(eb) and eb <= TOL_BF16
    assert np.isfinite(eS) and eS <= TOL_BF16
    rms_M = math.sqrt(float((Mo ** 2).mean()))
    if rms_M >= 0.1 / math.sqrt(D):  # M within 10x of the identity's scale: plain err/rms too
        eMp = rel_err(M, Mo)
        say(f"[summary] M err/rms={eMp:.3e}")
        assert eMp <= TOL_BF16


def test_summary_of_empty_run_is_identity():
    wl = CONFIGS[1].scaled(B=2, H=3, T=0)
    x = make_inputs(wl)
    M, b = _summary_gpu(x)
    assert torch.equal(M.cpu(), torch.eye(128).expand(2, 3, 128, 128))
    assert not b.cpu().any()


def _rand_summaries(P, B, H, D, seed):
    g = torch.Generator().manual_seed(seed)
    M = torch.randn(P, B, H, D, D, generator=g) / math.sqrt(D)
    b = torch.randn(P, B, H, D, D, generator=g)
    s0 = torch.randn(B, H, D, D, generator=g)
    return M, b, s0


@pytest.mark.parametrize("P,B,H,D", [(5, 2, 3, 128), (3, 1, 4, 64), (1, 1, 1, 128), (8, 1, 16, 128)])
def test_combine_matches_oracle(P, B, H, D):
    M, b, s0 = _rand_summaries(P, B, H, D, seed=P * 100 + D)
    say(f"[combine] P={P} B={B} H={H} D={D}")
    seg, fin = kda().combine_states(M.cuda(), b.cuda(), s0.cuda())
    torch.cuda.synchronize()
    sego, fino = oracle.combine(M.numpy(), b.numpy(), s0.numpy())
    es, ef = rel_err(seg, sego), rel_err(fin, fino)
    say(f"[combine] segment states err/rms={es:.3e} final err/rms={ef:.3e}")
    assert es <= TOL_F32 and ef <= TOL_F32
    assert torch.equal(seg[0].cpu(), s0)  # the first segment starts from the given state


def test_combine_without_segments_copies_and_may_alias():
    M, b, s0 = _rand_summaries(2, 1, 2, 64, seed=9)
    s = s0.cuda()
    _, fin = kda().combine_states(M[:0].cuda(), b[:0].cuda(), s, segment_states=False)
    torch.cuda.synchronize()
    assert torch.equal(fin.cpu(), s0)
    _, fin0 = kda().combine_states(M[:0].cuda(), b[:0].cuda(), None, segment_states=False)
    torch.cuda.synchronize()
    assert not fin0.cpu().any()
    # in place: final_state aliases initial_state
    kda().combine_states(M.cuda(), b.cuda(), s, segment_states=False, final_state=s)
    torch.cuda.synchronize()
    _, fino = oracle.combine(M.numpy(), b.numpy(), s0.numpy())
    assert rel_err(s, fino) <= TOL_F32


@pytest.mark.parametrize("wl_id,cuts", [
    (3, [0, 700, 1500, 2300, 3000]),   # floor stress recipe: 30 % of channels at the floor
    (2, [0, 64, 1100, 2049]),          # state in/out recipe, a first segment of one chunk
])
def test_context_parallel_split_matches_whole(wl_id, cuts):
    """The pages' context-parallel flow on one GPU: summarise each segment on its own,
    combine the summaries in order, re-run every segment from its incoming state;
    outputs and final state must match one oracle pass over the whole sequence."""
    T = cuts[-1]
    wl = CONFIGS[wl_id].scaled(B=1, H=4, T=T, init_state=True)
    x = make_inputs(wl, seed=50 + wl_id)
    say(f"[kcp] recipe {wl.name} T={T} cuts={cuts}")
    xs = {k: x[k].cuda() for k in KEYS}
    s0 = x["initial_state"].cuda()
    sl = lambda t, lo, hi: t[:, lo:hi].contiguous()
    Ms, bs = [], []
    for lo, hi in zip(cuts, cuts[1:]):
        M, b = kda().chunk_summary(*(sl(xs[k], lo, hi) for k in ("k", "v", "log_alpha", "beta")))
        Ms.append(M)
        bs.append(b)
    seg, fin = kda().combine_states(torch.stack(Ms), torch.stack(bs), s0)
    ys = []
    for p, (lo, hi) in enumerate(zip(cuts, cuts[1:])):
        y, _ = kda().chunk_fwd(*(sl(xs[k], lo, hi) for k in KEYS), initial_state=seg[p].contiguous())
        ys.append(y)
    torch.cuda.synchronize()
    yo, so = oracle.fwd(*(x[k] for k in KEYS), initial_state=x["initial_state"])
    ey, es = rel_err(torch.cat(ys, dim=1), yo), rel_err(fin, so)
    say(f"[kcp] y err/rms={ey:.3e} final state err/rms={es:.3e}")
    assert np.isfinite(ey) and ey <= TOL_BF16
    assert np.isfinite(es) and es <= TOL_BF16


@pytest.mark.parametrize("H,T", [(4, 1000), (1, 8192)])
def test_rerun_takes_the_summary_cards(H, T):
    """A summary given q leaves complete cards; the forward that takes them (card builder
    skipped) is bit for bit the forward that builds them (T = 8192, H = 1 also takes
    the segment scan)."""
    wl = CONFIGS[3].scaled(B=1, H=H, T=T, init_state=True)
    x = {k: v.cuda() for k, v in make_inputs(wl, seed=300 + T).items() if v is not None}
    ws = torch.empty(kda().workspace_bytes(1, T, H, 128), dtype=torch.uint8, device="cuda")
    y0, s0 = kda().chunk_fwd(*(x[k] for k in KEYS), initial_state=x["initial_state"], output_final_state=True)
    M, b = kda().chunk_summary(x["k"], x["v"], x["log_alpha"], x["beta"], q=x["q"], workspace=ws)
    y1, s1 = kda().chunk_fwd(*(x[k] for k in KEYS), initial_state=x["initial_state"], output_final_state=True,
                             workspace=ws, cards_ready=True)
    torch.cuda.synchronize()
    say(f"[kcp] cards reused H={H} T={T}: identical y {torch.equal(y0, y1)}, final {torch.equal(s0, s1)}")
    assert torch.equal(y0, y1) and torch.equal(s0, s1)


# The general path (fp32 inputs, or chunks of 16 / 32 tokens): its cards and one state
# pass per (b, h) that carries b from zero and M from the identity.  Same error measures;
# the fp32 bound for fp32 inputs.
GENERAL = [
    # (dtype, D, chunk, T, alpha_mu, beta_mu)
    ("f32", 64, 0, 300, 2.0, 0.0),
    ("f32", 128, 32, 257, 6.0, 0.0),
    ("f32", 128, 16, 100, 7.0, -3.0),
    ("bf16", 128, 16, 300, 2.0, 0.0),
    ("bf16", 64, 32, 190, 6.0, -3.0),
]


@pytest.mark.parametrize("dtype,D,chunk,T,alpha_mu,beta_mu", GENERAL,
                         ids=[f"{g[0]} d{g[1]} chunk {g[2] or 16} T{g[3]}" for g in GENERAL])
def test_summary_general_path_matches_oracle(dtype, D, chunk, T, alpha_mu, beta_mu):
    wl = CONFIGS[1].scaled(B=1, H=2, T=T, Dk=D, Dv=D, dtype=dtype, alpha_mu=alpha_mu, beta_mu=beta_mu,
                           init_state=True)
    x = make_inputs(wl, seed=60 + T)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    say(f"[summary general] {dtype} D={D} chunk={chunk} T={T} alpha_mu={alpha_mu} beta_mu={beta_mu}")
    d = {k: x[k].cuda() for k in ("k", "v", "log_alpha", "beta")}
    M, b = kda().chunk_summary(d["k"], d["v"], d["log_alpha"], d["beta"], chunk=chunk)
    torch.cuda.synchronize()
    Mo, bo = oracle.summary(x["k"], x["v"], x["log_alpha"], x["beta"])
    eM, eb = rel_err(M, Mo, floor=1 / math.sqrt(D)), rel_err(b, bo)
    s0 = x["initial_state"].double().numpy() * 50
    _, so = oracle.fwd(*(x[k] for k in KEYS), initial_state=s0)
    eS = rel_err(np.matmul(_np(M), s0) + _np(b), so)
    say(f"[summary general] M err={eM:.3e} b err/rms={eb:.3e} M S0 + b err/rms={eS:.3e} (tol {tol})")
    assert np.isfinite(eM) and eM <= tol
    assert np.isfinite(eb) and eb <= tol
    assert np.isfinite(eS) and eS <= tol
