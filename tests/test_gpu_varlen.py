"""GPU parity of the variable-length batch and the block-granular state snapshots
(through the C ABI) against the fp64 oracle.

Page "Kimi K3 report walk-through", section on RL infrastructure and the prefix
cache of linear attention: the state is kept at block granularity, so a cached
prefix can be continued.  The oracle needs nothing new: every packed sequence is
an independent run (oracle.fwd on it alone), and a snapshot is the state the
oracle reaches after that many tokens of the sequence.  Error measure and limit as
for kda_chunk_fwd: max |gpu - oracle| / rms(oracle) <= 2e-2 (bf16 inputs).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from kda_workloads import CONFIGS, make_inputs, make_raw_inputs

pytestmark = pytest.mark.gpu

TOL = 2e-2
KEYS = ("q", "k", "v", "log_alpha", "beta", "gate")


def kda():
    import gated_delta_rule_106_amd as m
    return m


def say(*a):
    print(*a, flush=True)


def rel_err(got, ref):
    got = got.detach().double().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    return float(np.abs(got - ref).max()) / max(math.sqrt(float((ref ** 2).mean())), 1e-30)


def packed(lengths, H, D, seed, wl_id=2, raw=False, pad_rows=0):
    """Sequences of the given lengths from one recipe, packed along rows (plus unused
    trailing rows), with per-sequence initial states."""
    rows = sum(lengths) + pad_rows
    wl = CONFIGS[wl_id].scaled(B=1, H=H, T=rows, Dk=D, Dv=D, init_state=False)
    x = (make_raw_inputs if raw else make_inputs)(wl, seed=seed)
    x = {k: x[k][0] for k in KEYS}  # [rows, H, D]
    g = torch.Generator().manual_seed(seed)
    s0 = torch.randn(len(lengths), H, D, D, generator=g) * 0.02
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return x, s0, cu


def run(x, s0, cu, snapshot_every=0, **opts):
    d = {k: x[k].cuda() for k in KEYS}
    y, fin, snaps = kda().chunk_fwd_varlen(*(d[k] for k in KEYS), torch.from_numpy(cu).cuda(),
                                           initial_state=s0.cuda(), output_final_state=True,
                                           snapshot_every=snapshot_every, **opts)
    torch.cuda.synchronize()
    return y, fin, snaps


def oracle_seq(x, s0, cu, i, upto=None, **opts):
    lo, hi = int(cu[i]), int(cu[i + 1])
    if upto is not None:
        hi = lo + upto
    xs = {k: x[k][lo:hi].unsqueeze(0).contiguous() for k in KEYS}
    return oracle.fwd(*(xs[k] for k in KEYS), initial_state=s0[i:i + 1], **opts)


@pytest.mark.parametrize("D", [64, 128])
def test_varlen_matches_oracle_per_sequence(D):
    lengths = [0, 1, 63, 64, 65, 700, 130]
    x, s0, cu = packed(lengths, 3, D, seed=200 + D)
    say(f"[varlen] D={D} lengths={lengths}")
    y, fin, _ = run(x, s0, cu)
    for i in range(len(lengths)):
        yo, so = oracle_seq(x, s0, cu, i)
        ey = rel_err(y[cu[i]:cu[i + 1]], yo[0])
        es = rel_err(fin[i], so[0])
        say(f"[varlen] seq {i} len {lengths[i]}: y err/rms={ey:.3e} final err/rms={es:.3e}")
        assert ey <= TOL and es <= TOL


def test_equal_lengths_bitwise_equal_to_batch():
    """cu = i T over a [N, T, H, D] batch is the same memory: the results are the
    batch call's, bit for bit (the same card arithmetic, another card order)."""
    N, T, H = 3, 300, 2
    wl = CONFIGS[2].scaled(B=N, H=H, T=T)
    x = {k: v.cuda() for k, v in make_inputs(wl, seed=210).items() if v is not None}
    s0 = x["initial_state"]
    yb, sb = kda().chunk_fwd(*(x[k] for k in KEYS), initial_state=s0, output_final_state=True)
    cu = torch.arange(0, (N + 1) * T, T, dtype=torch.int64, device="cuda")
    flat = {k: x[k].reshape(N * T, *x[k].shape[2:]) for k in KEYS}
    yv, sv, _ = kda().chunk_fwd_varlen(*(flat[k] for k in KEYS), cu, initial_state=s0, output_final_state=True)
    torch.cuda.synchronize()
    say("[varlen] equal lengths vs batch: identical y", torch.equal(yv.reshape(N, T, H, -1), yb),
        "identical final", torch.equal(sv, sb))
    assert torch.equal(yv.reshape(N, T, H, -1), yb) and torch.equal(sv, sb)


@pytest.mark.parametrize("every", [64, 128])
def test_snapshots_match_oracle_prefix_states(every):
    lengths = [700, 130, 0, 256, 64]
    x, s0, cu = packed(lengths, 2, 128, seed=220 + every, wl_id=3)
    say(f"[snap] every={every} lengths={lengths}")
    y, fin, snaps = run(x, s0, cu, snapshot_every=every)
    assert snaps.shape[0] == sum(lengths) // every + len(lengths)
    worst = 0.0
    for i, L in enumerate(lengths):
        for kk in range(L // every):
            slot = kda().snapshot_slot(cu, i, kk, every)
            _, so = oracle_seq(x, s0, cu, i, upto=(kk + 1) * every)
            e = rel_err(snaps[slot], so[0])
            worst = max(worst, e)
            assert e <= TOL, (i, kk, e)
    say(f"[snap] every={every}: worst snapshot err/rms={worst:.3e}")


def test_continuing_from_a_snapshot_reproduces_the_rest():
    """Prefix cache: the state cached after P tokens continues the sequence exactly as
    the whole run does."""
    lengths = [900, 333]
    x, s0, cu = packed(lengths, 2, 128, seed=230)
    y, fin, snaps = run(x, s0, cu, snapshot_every=256)
    i, kk = 0, 2  # after 768 tokens of sequence 0
    p = (kk + 1) * 256
    slot = kda().snapshot_slot(cu, i, kk, 256)
    rest = {k: x[k][p:lengths[0]].unsqueeze(0).contiguous().cuda() for k in KEYS}
    y2, s2 = kda().chunk_fwd(*(rest[k] for k in KEYS), initial_state=snaps[slot:slot + 1].contiguous(),
                             output_final_state=True)
    torch.cuda.synchronize()
    yo, so = oracle_seq(x, s0, cu, 0)
    ey, es = rel_err(y2[0], yo[0, p:]), rel_err(s2[0], so[0])
    say(f"[snap] continuation from token {p}: y err/rms={ey:.3e} final err/rms={es:.3e}")
    assert ey <= TOL and es <= TOL


def test_rows_outside_the_sequences_are_left_alone():
    lengths = [100, 50]
    x, s0, cu = packed(lengths, 2, 64, seed=240, pad_rows=40)
    d = {k: x[k].cuda() for k in KEYS}
    out = torch.full((sum(lengths) + 40, 2, 64), 7.0, device="cuda")
    y, fin, _ = kda().chunk_fwd_varlen(*(d[k] for k in KEYS), torch.from_numpy(cu).cuda(),
                                       initial_state=s0.cuda(), output_final_state=True, out=out)
    torch.cuda.synchronize()
    assert torch.equal(y[150:].cpu(), torch.full((40, 2, 64), 7.0))
    for i in range(2):
        yo, so = oracle_seq(x, s0, cu, i)
        assert rel_err(y[cu[i]:cu[i + 1]], yo[0]) <= TOL and rel_err(fin[i], so[0]) <= TOL


def test_varlen_with_fused_preparation():
    lengths = [77, 300, 1]
    x, s0, cu = packed(lengths, 2, 128, seed=250, raw=True)
    opts = dict(qk_norm=True, gate_logits=True)
    y, fin, _ = run(x, s0, cu, **opts)
    for i in range(len(lengths)):
        yo, so = oracle_seq(x, s0, cu, i, **opts)
        ey, es = rel_err(y[cu[i]:cu[i + 1]], yo[0]), rel_err(fin[i], so[0])
        say(f"[varlen] fused seq {i}: y err/rms={ey:.3e} final err/rms={es:.3e}")
        assert ey <= TOL and es <= TOL


def test_many_short_sequences():
    """300 sequences (the sequence map spans two 256-entry blocks, and N H >= 64 takes the
    two-value-tile state pass), lengths 0 .. 150 with a sample compared to the oracle,
    snapshots every 64 tokens on the sampled sequences."""
    g = np.random.default_rng(260)
    lengths = [int(x) for x in g.integers(0, 151, 300)]
    lengths[5] = 0
    lengths[299] = 150
    x, s0, cu = packed(lengths, 2, 128, seed=260)
    say(f"[varlen] 300 sequences, {sum(lengths)} tokens")
    y, fin, snaps = run(x, s0, cu, snapshot_every=64)
    worst = 0.0
    for i in (0, 1, 5, 17, 128, 255, 256, 257, 298, 299):
        yo, so = oracle_seq(x, s0, cu, i)
        ey, es = rel_err(y[cu[i]:cu[i + 1]], yo[0]), rel_err(fin[i], so[0])
        worst = max(worst, ey, es)
        assert ey <= TOL and es <= TOL, (i, ey, es)
        for kk in range(lengths[i] // 64):
            _, sp = oracle_seq(x, s0, cu, i, upto=(kk + 1) * 64)
            assert rel_err(snaps[kda().snapshot_slot(cu, i, kk, 64)], sp[0]) <= TOL
    say(f"[varlen] 300 sequences: worst sampled err/rms={worst:.3e}")


def test_full_size_batch_as_varlen_bitwise():
    """B2 H32 T8192 (the state in/out workload at full size) as two packed sequences:
    outputs and final states are the batch call's bit for bit, and the snapshot after
    4096 tokens is bit for bit the batch call's final state over that prefix (the same
    cards and arithmetic either way)."""
    wl = CONFIGS[2]
    x = {k: v.cuda() for k, v in make_inputs(wl).items() if v is not None}
    B, T, H = wl.B, wl.T, wl.H
    yb, sb = kda().chunk_fwd(*(x[k] for k in KEYS), initial_state=x["initial_state"], output_final_state=True)
    cu = torch.arange(0, (B + 1) * T, T, dtype=torch.int64, device="cuda")
    flat = {k: x[k].reshape(B * T, *x[k].shape[2:]) for k in KEYS}
    yv, sv, snaps = kda().chunk_fwd_varlen(*(flat[k] for k in KEYS), cu, initial_state=x["initial_state"],
                                           output_final_state=True, snapshot_every=4096)
    half = {k: x[k][:, :4096].contiguous() for k in KEYS}
    _, sh = kda().chunk_fwd(*(half[k] for k in KEYS), initial_state=x["initial_state"], output_final_state=True)
    torch.cuda.synchronize()
    same_y, same_s = torch.equal(yv.reshape(B, T, H, -1), yb), torch.equal(sv, sb)
    same_snap = all(torch.equal(snaps[kda().snapshot_slot(cu.cpu(), i, 0, 4096)], sh[i]) for i in range(B))
    last = all(torch.equal(snaps[kda().snapshot_slot(cu.cpu(), i, 1, 4096)], sb[i]) for i in range(B))
    say(f"[varlen] full size B2 H32 T8192: y {same_y}, final {same_s}, snapshot@4096 {same_snap}, @8192 {last}")
    assert same_y and same_s and same_snap and last


def test_sequences_may_start_after_row_zero():
    """cu[0] > 0: the rows before the first sequence are not read and out is not written
    there, exactly as for rows after the last one."""
    lengths = [90, 0, 33]
    x, s0, cu = packed(lengths, 2, 128, seed=270, pad_rows=50)
    rows = sum(lengths) + 50
    shift = 20  # sequences at rows 20 .. 143; rows 0..19 and 143.. are outside
    xs = {k: torch.roll(x[k], shifts=shift, dims=0) for k in KEYS}
    cu2 = cu + shift
    d = {k: xs[k].cuda() for k in KEYS}
    out = torch.full((rows, 2, 128), -3.0, device="cuda")
    y, fin, _ = kda().chunk_fwd_varlen(*(d[k] for k in KEYS), torch.from_numpy(cu2).cuda(),
                                       initial_state=s0.cuda(), output_final_state=True, out=out)
    torch.cuda.synchronize()
    assert torch.equal(y[:shift].cpu(), torch.full((shift, 2, 128), -3.0))
    assert torch.equal(y[int(cu2[-1]):].cpu(), torch.full((rows - int(cu2[-1]), 2, 128), -3.0))
    for i in range(len(lengths)):
        yo, so = oracle_seq(x, s0, cu, i)
        assert rel_err(y[cu2[i]:cu2[i + 1]], yo[0]) <= TOL and rel_err(fin[i], so[0]) <= TOL
    say("[varlen] sequences starting at row 20: outside rows untouched, parity held")


# The general path (fp32 inputs, or chunks of 16 / 32 tokens): the same sequence map
# places its cards and its state pass.  Limits as for kda_chunk_fwd: 1e-4 for fp32
# inputs, 2e-2 for bf16.
GENERAL = [
    # (dtype, D, chunk, workload of the recipe)
    (torch.float32, 64, 0, 0),
    (torch.float32, 128, 32, 0),
    (torch.bfloat16, 128, 16, 2),
    (torch.bfloat16, 64, 32, 2),
]


@pytest.mark.parametrize("dtype,D,chunk,wl_id", GENERAL,
                         ids=[f"{'fp32' if g[0] == torch.float32 else 'bf16'} d{g[1]} chunk {g[2] or 16}"
                              for g in GENERAL])
def test_varlen_general_path_matches_oracle(dtype, D, chunk, wl_id):
    """Empty, one-token, ragged and exact-chunk sequences, with snapshots every 64
    tokens, against the oracle run on each sequence alone."""
    lengths = [0, 1, 15, 16, 17, 200, 0, 65, 128]
    x, s0, cu = packed(lengths, 2, D, seed=240 + D + chunk, wl_id=wl_id)
    x = {k: v.to(dtype) for k, v in x.items()}
    tol = 1e-4 if dtype == torch.float32 else TOL
    say(f"[varlen general] {dtype} D={D} chunk={chunk} lengths={lengths}")
    y, fin, snaps = run(x, s0, cu, snapshot_every=64, chunk=chunk)
    worst = 0.0
    for i, L in enumerate(lengths):
        yo, so = oracle_seq(x, s0, cu, i)
        ey, es = rel_err(y[cu[i]:cu[i + 1]], yo[0]), rel_err(fin[i], so[0])
        worst = max(worst, ey, es)
        assert ey <= tol and es <= tol, (i, ey, es)
        for kk in range(L // 64):
            _, sk = oracle_seq(x, s0, cu, i, upto=(kk + 1) * 64)
            e = rel_err(snaps[kda().snapshot_slot(cu, i, kk, 64)], sk[0])
            worst = max(worst, e)
            assert e <= tol, (i, kk, e)
    say(f"[varlen general] worst err/rms over outputs, final states and snapshots: {worst:.3e}")


def test_varlen_general_path_equal_lengths_bitwise_equal_to_batch():
    """fp32, chunk 16: cu = i T over a [N, T, H, D] batch gives the batch call's
    results bit for bit."""
    N, T, H = 3, 100, 2
    wl = CONFIGS[0].scaled(B=N, H=H, T=T, init_state=True)
    x = {k: v.cuda() for k, v in make_inputs(wl, seed=250).items() if v is not None}
    s0 = x["initial_state"]
    yb, sb = kda().chunk_fwd(*(x[k] for k in KEYS), initial_state=s0, output_final_state=True, chunk=16)
    cu = torch.arange(0, (N + 1) * T, T, dtype=torch.int64, device="cuda")
    flat = {k: x[k].reshape(N * T, *x[k].shape[2:]) for k in KEYS}
    yv, sv, _ = kda().chunk_fwd_varlen(*(flat[k] for k in KEYS), cu, initial_state=s0, output_final_state=True,
                                       chunk=16)
    torch.cuda.synchronize()
    assert torch.equal(yv.reshape(N, T, H, -1), yb) and torch.equal(sv, sb)
    say("[varlen general] equal lengths vs batch: identical")
