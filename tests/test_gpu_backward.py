"""GPU parity of the chunkwise backward pass (kda_chunk_bwd, through the C ABI)
against the oracle's reverse mode through the token steps (kda_oracle_bwd).

The loss is L = sum(d_out * y) + sum(d_final_state * S_T); the gradients are
taken with respect to q, k, v, log alpha, beta, the gate logits and the initial
state (page "3T models are no longer magic", section "Gate 1: KDA makes it
computable", in reverse; the GPU side works chunk by chunk, page "Kimi K3 report
walk-through", section "Compute paradigm").

Error measure: max |gpu - oracle| / rms(oracle) over each gradient tensor.  Both
sides read the same input bits and the GPU side computes every step in fp32 (the
oracle in fp64), so the bound is the one the forward is held to for fp32
arithmetic, 1e-4 of the RMS, for either input dtype.  fp32 rounding of the sums
over a 64-token chunk and 128 channels, carried through the non-expansive
recurrence, stays well below it (the largest error measured over these cases is
about 3e-5); a dropped or misplaced term moves a gradient by a sizeable fraction
of its RMS.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from kda_workloads import CONFIGS, make_inputs, make_raw_inputs, small

pytestmark = pytest.mark.gpu

TOL = 1e-4
KEYS = ("q", "k", "v", "log_alpha", "beta", "gate")
GRADS = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dgate", "dinitial_state")


def kda():
    import gated_delta_rule_106_amd as m
    return m


def say(*a):
    print(*a, flush=True)


def rel_err(got, ref):
    got = got.detach().double().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    rms = math.sqrt(float((ref ** 2).mean()))
    return float(np.abs(got - ref).max()) / max(rms, 1e-30)


def _cotangents(wl, seed, with_dst):
    g = torch.Generator().manual_seed(seed)
    dy = torch.randn((wl.B, wl.T, wl.H, wl.Dv), generator=g).to(wl.torch_dtype)
    dst = torch.randn((wl.B, wl.H, wl.Dk, wl.Dv), generator=g) * 0.1 if with_dst else None
    return dy, dst


def _run(x, dy, dst, clamp=True, **opts):
    d = {n: x[n].cuda() for n in KEYS}
    s0 = x["initial_state"].cuda() if x.get("initial_state") is not None else None
    g = kda().chunk_bwd(*(d[n] for n in KEYS), dy.cuda(), initial_state=s0,
                        d_final_state=dst.cuda() if dst is not None else None, clamp=clamp, **opts)
    torch.cuda.synchronize()
    return g


def _oracle(x, dy, dst, clamp=True, **opts):
    return oracle.bwd(*(x[n] for n in KEYS), dy.double().numpy(), initial_state=x.get("initial_state"),
                      d_final_state=dst, clamp=clamp, **opts)


def _check(tag, g, ref):
    errs = {n: rel_err(g[n], ref[n]) for n in GRADS}
    say(f"[bwd] {tag}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= TOL, (tag, n, e)


CASES = [
    # (tag, workload, initial state, d_final_state)
    ("bf16 d64 T150 (ragged tail) state in, dS_T", small(CONFIGS[2], B=1, H=2, T=150, Dk=64, Dv=64), True, True),
    ("fp32 d128 B2 T64 (one chunk)", small(CONFIGS[0], B=2, H=1, T=64, Dk=128, Dv=128, chunk=64), False, False),
    ("bf16 d128 T200 floor channels, dS_T", small(CONFIGS[3], H=2, T=200), False, True),
    ("bf16 d128 T1", small(CONFIGS[2], B=2, H=1, T=1), True, True),
    ("fp32 d64 T300 state in", small(CONFIGS[0], B=1, H=2, T=300, init_state=True), True, False),
    ("fp32 d128 T230 (ragged tail) state in, dS_T",
     small(CONFIGS[0], B=1, H=2, T=230, Dk=128, Dv=128, chunk=64), True, True),
]


@pytest.mark.parametrize("tag,wl,init,with_dst", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(tag, wl, init, with_dst):
    say(f"[bwd] case {tag}: B{wl.B} H{wl.H} T{wl.T} d{wl.Dk} {wl.dtype}")
    x = make_inputs(wl.scaled(init_state=init))
    dy, dst = _cotangents(wl, 11 + wl.T, with_dst)
    g = _run(x, dy, dst)
    _check(tag, g, _oracle(x, dy, dst))


def test_backward_is_deterministic():
    wl = small(CONFIGS[2], B=1, H=2, T=150, Dk=64, Dv=64)
    x = make_inputs(wl)
    dy, dst = _cotangents(wl, 5, True)
    a, b = _run(x, dy, dst), _run(x, dy, dst)
    for n in GRADS:
        assert torch.equal(a[n], b[n]), n
    say("[bwd] two calls agree bit for bit")


@pytest.mark.parametrize("clamp", [True, False])
def test_clamp_gradient(clamp):
    """log alpha outside [ln 0.0067, 0]: with the clamp its gradient is zero there and the
    other gradients see the clamped value; without it the raw value is used throughout."""
    wl = small(CONFIGS[0], B=1, H=2, T=100, Dk=64, Dv=64, chunk=64)
    x = make_inputs(wl)
    la = x["log_alpha"].clone()
    gen = torch.Generator().manual_seed(3)
    pick = torch.rand(la.shape, generator=gen)
    la[pick < 0.05] = -6.5
    la[pick > 0.97] = 0.05
    x["log_alpha"] = la.contiguous()
    dy, dst = _cotangents(wl, 7, True)
    g = _run(x, dy, dst, clamp=clamp)
    ref = _oracle(x, dy, dst, clamp=clamp)
    _check(f"clamp={clamp}", g, ref)
    if clamp:
        dead = (la < math.log(0.0067)) | (la > 0)
        assert dead.any() and bool((g["dlog_alpha"].cpu()[dead] == 0).all())


def test_empty_sequence_passes_the_state_gradient_through():
    wl = small(CONFIGS[2], B=2, H=3, T=0, Dk=64, Dv=64)
    x = make_inputs(wl)
    _, dst = _cotangents(small(wl, T=1), 1, True)
    g = _run(x, torch.zeros((2, 0, 3, 64), dtype=torch.bfloat16), dst)
    assert torch.equal(g["dinitial_state"].cpu(), dst)
    g = _run(x, torch.zeros((2, 0, 3, 64), dtype=torch.bfloat16), None)
    assert not g["dinitial_state"].cpu().any()
    say("[bwd] T=0: the state gradient passes through unchanged")


def test_full_size_headline_sampled_heads():
    """B1 H8 T4096 d128 bf16 (the headline prefill shape) in the launch configuration
    the bench times; heads are independent, so the oracle runs on two of them."""
    wl = CONFIGS[1]
    x = make_inputs(wl)
    dy, _ = _cotangents(wl, 21, False)
    g = _run(x, dy, None)
    for h in (0, 5):
        xs = {n: x[n][:, :, h:h + 1].contiguous() for n in KEYS}
        ref = _oracle(xs, dy[:, :, h:h + 1].contiguous(), None)
        gh = {n: (g[n][:, :, h:h + 1] if n != "dinitial_state" else g[n][:, h:h + 1]) for n in GRADS}
        _check(f"B1 H8 T4096 d128 bf16, head {h}", gh, ref)


def test_more_chunks_than_workgroups():
    """520 chunks on at most 512 workgroups: some workgroups take two chunks, and the
    gradient kernel recomputes the shared per-chunk steps instead of reusing the prep's."""
    wl = small(CONFIGS[2], B=1, H=2, T=260 * 64, Dk=64, Dv=64)
    x = make_inputs(wl)
    dy, dst = _cotangents(wl, 31, True)
    _check("B1 H2 T16640 d64 bf16 (520 chunks)", _run(x, dy, dst), _oracle(x, dy, dst))


def test_full_size_state_in_out_sampled_units():
    """B2 H32 T8192 d128 bf16 with an initial state and dS_T: 8192 chunks over 512
    workgroups (the recompute path); (batch, head) units are independent, so the oracle
    runs on two of them."""
    wl = CONFIGS[2]
    x = make_inputs(wl)
    dy, dst = _cotangents(wl, 41, True)
    g = _run(x, dy, dst)
    for b, h in ((0, 3), (1, 17)):
        xs = {n: x[n][b:b + 1, :, h:h + 1].contiguous() for n in KEYS}
        xs["initial_state"] = x["initial_state"][b:b + 1, h:h + 1].contiguous()
        ref = _oracle(xs, dy[b:b + 1, :, h:h + 1].contiguous(), dst[b:b + 1, h:h + 1].contiguous())
        gh = {n: (g[n][b:b + 1, :, h:h + 1] if n != "dinitial_state" else g[n][b:b + 1, h:h + 1]) for n in GRADS}
        _check(f"B2 H32 T8192 d128 bf16 state in/out, unit (b={b}, h={h})", gh, ref)


def test_without_initial_state_gradient():
    """d_initial_state NULL (the launch configuration the bench times): every other
    gradient is bit for bit the one of a call that also returns dS0."""
    wl = small(CONFIGS[2], B=1, H=2, T=150, Dk=64, Dv=64)
    x = make_inputs(wl)
    dy, dst = _cotangents(wl, 51, True)
    d = {n: x[n].cuda() for n in KEYS}
    s0, dstc, dyc = x["initial_state"].cuda(), dst.cuda(), dy.cuda()
    full = kda().chunk_bwd(*(d[n] for n in KEYS), dyc, initial_state=s0, d_final_state=dstc)
    part = kda().chunk_bwd(*(d[n] for n in KEYS), dyc, initial_state=s0, d_final_state=dstc,
                           need_initial_state_grad=False)
    torch.cuda.synchronize()
    assert part["dinitial_state"] is None
    for n in GRADS[:-1]:
        assert torch.equal(full[n], part[n]), n
    say("[bwd] without dS0: the other gradients are unchanged")


# The fused preparation (page "3T models are no longer magic", section "FlashKDA": the
# Q and K normalisation and the forget-gate computation belong to the preparation
# step): raw q and k, forget-gate logits, the gradients taken with respect to them.
# Raw inputs: each token's q and k scaled by a random factor in [0.1, 10); channels
# at the floor carry logits of -12 (log-sigmoid below ln 0.0067: clamped, zero gradient).
PREP = dict(qk_norm=True, gate_logits=True)
PREP_CASES = [
    ("bf16 d128 T200 (ragged tail) state in, dS_T", small(CONFIGS[3], H=2, T=200), True, True),
    ("fp32 d64 T150 state in", small(CONFIGS[0], B=1, H=2, T=150, Dk=64, Dv=64, chunk=64), True, False),
    ("bf16 d64 T64 (one chunk), dS_T", small(CONFIGS[2], B=2, H=1, T=64, Dk=64, Dv=64), False, True),
    ("fp32 d128 T130 state in, dS_T", small(CONFIGS[0], B=1, H=1, T=130, Dk=128, Dv=128, chunk=64), True, True),
]


@pytest.mark.parametrize("tag,wl,init,with_dst", PREP_CASES, ids=[c[0] for c in PREP_CASES])
def test_backward_with_fused_preparation(tag, wl, init, with_dst):
    say(f"[bwd] prepared case {tag}: B{wl.B} H{wl.H} T{wl.T} d{wl.Dk} {wl.dtype}")
    x = make_raw_inputs(wl.scaled(init_state=init), seed=200 + wl.T)
    dy, dst = _cotangents(wl, 13 + wl.T, with_dst)
    g = _run(x, dy, dst, **PREP)
    ref = _oracle(x, dy, dst, **PREP)
    _check("prepared " + tag, g, ref)
    dead = x["log_alpha"].float() < -11.0  # the floor channels' logits
    if dead.any():
        assert bool((g["dlog_alpha"].cpu()[dead] == 0).all())


@pytest.mark.parametrize("opts", [dict(qk_norm=True), dict(gate_logits=True),
                                  dict(gate_logits=True, clamp=False)],
                         ids=["qk_norm", "gate_logits", "gate_logits no clamp"])
def test_backward_each_preparation_option(opts):
    """One option on, the other input arriving prepared.  Without the clamp the recipe
    has no floor channels (the logits keep the decay within the exponent range)."""
    clamp = opts.pop("clamp", True)
    wl = small(CONFIGS[1], B=1, H=2, T=170)
    if not clamp:
        wl = wl.scaled(floor_frac=0.0)
    raw, x = make_raw_inputs(wl, seed=97), make_inputs(wl, seed=97)
    if opts.get("qk_norm"):
        x["q"], x["k"] = raw["q"], raw["k"]
    if opts.get("gate_logits"):
        x["log_alpha"] = raw["log_alpha"]
    dy, dst = _cotangents(wl, 19, True)
    _check(f"option {opts} clamp={clamp}", _run(x, dy, dst, clamp=clamp, **opts),
           _oracle(x, dy, dst, clamp=clamp, **opts))


def test_backward_fused_preparation_full_size_sampled_heads():
    """B1 H8 T4096 d128 bf16 with raw q, k and logits; heads are independent, so the
    oracle runs on two of them."""
    wl = CONFIGS[1]
    x = make_raw_inputs(wl, seed=23)
    dy, _ = _cotangents(wl, 29, False)
    g = _run(x, dy, None, **PREP)
    for h in (2, 7):
        xs = {n: x[n][:, :, h:h + 1].contiguous() for n in KEYS}
        ref = _oracle(xs, dy[:, :, h:h + 1].contiguous(), None, **PREP)
        gh = {n: (g[n][:, :, h:h + 1] if n != "dinitial_state" else g[n][:, h:h + 1]) for n in GRADS}
        _check(f"prepared B1 H8 T4096 d128 bf16, head {h}", gh, ref)
