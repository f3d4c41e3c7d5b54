"""The entry points under HIP graph capture: a prefill, a decode step and a backward
pass captured once into one graph (through torch.cuda.CUDAGraph, on the capturing
stream the binding passes to the C ABI) and replayed on fresh inputs copied into the
captured tensors.  Every replay, with eager work and synchronisations between the
replays, must equal the eager calls on the same inputs bit for bit (the kernels are
deterministic and the graph replays the same launches).  The library issues no memory
set, allocation or synchronisation of its own, so nothing else is recorded.
"""
import pytest
import torch

from kda_workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

KEYS = ("q", "k", "v", "log_alpha", "beta", "gate")


def kda():
    import gated_delta_rule_106_amd as m
    return m


def say(*a):
    print(*a, flush=True)


def _fresh(wl, seed):
    x = make_inputs(wl, seed=seed)
    g = torch.Generator().manual_seed(seed + 1)
    dy = torch.randn((wl.B, wl.T, wl.H, wl.Dv), generator=g).to(wl.torch_dtype)
    return x, dy


def test_prefill_decode_backward_replay_in_a_graph():
    wl = CONFIGS[1].scaled(B=1, H=4, T=700, init_state=True)
    dec = CONFIGS[4].scaled(B=3, H=4)
    say("[graph] prefill B1 H4 T700, decode B3 H4, backward B1 H4 T700")
    x, dy = _fresh(wl, 5)
    xd = make_inputs(dec, seed=6)
    # static (captured) tensors
    s = {n: x[n].cuda() for n in KEYS}
    s0 = x["initial_state"].cuda()
    sdy = dy.cuda()
    sd = {n: xd[n].cuda() for n in KEYS}
    sstate = xd["state"].cuda().clone()
    out = torch.empty((wl.B, wl.T, wl.H, wl.Dv), dtype=torch.float32, device="cuda")
    fin = torch.empty_like(s0)
    ws = torch.empty(kda().workspace_bytes(wl.B, wl.T, wl.H, wl.Dk), dtype=torch.uint8, device="cuda")
    ydec = torch.empty((dec.B, dec.H, dec.Dv), dtype=torch.float32, device="cuda")

    def work():
        kda().chunk_fwd(*(s[n] for n in KEYS), initial_state=s0, out=out, final_state=fin, workspace=ws,
                        output_final_state=True)
        kda().decode_step(*(sd[n] for n in KEYS), state=sstate, out=ydec)
        return kda().chunk_bwd(*(s[n] for n in KEYS), sdy, initial_state=s0)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture (loads the library, sets attributes)
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    state_before = sstate.clone()
    with torch.cuda.graph(graph):
        grads = work()
    torch.cuda.synchronize()
    sstate.copy_(state_before)  # capture did not run the step; restore for clarity
    for rep in range(3):
        x, dy = _fresh(wl, 100 + rep)
        xd = make_inputs(dec, seed=200 + rep)
        for n in KEYS:
            s[n].copy_(x[n])
            sd[n].copy_(xd[n])
        s0.copy_(x["initial_state"])
        sdy.copy_(dy)
        start = xd["state"].cuda()
        sstate.copy_(start)
        graph.replay()
        torch.cuda.synchronize()
        got = (out.clone(), fin.clone(), ydec.clone(), sstate.clone(), {k: v.clone() for k, v in grads.items()
                                                                        if v is not None})
        # eager on the same inputs
        sstate.copy_(start)
        ref_grads = work()
        torch.cuda.synchronize()
        assert torch.equal(got[0], out) and torch.equal(got[1], fin), rep
        assert torch.equal(got[2], ydec) and torch.equal(got[3], sstate), rep
        for k, v in got[4].items():
            assert torch.equal(v, ref_grads[k]), (rep, k)
        say(f"[graph] replay {rep}: prefill, decode and backward equal the eager calls bit for bit")
