"""kda_chunk_fwd_noalloc (the entry point for callers that cannot allocate device
memory) against kda_chunk_fwd, through the C ABI, on consecutive calls that share the
library's fixed scratch: first B1 H8 T4096 d128 bf16 (512 cards), then smaller
calls whose cards land on what the first one left there.  Both entry points run
the same kernels on the same inputs, so the outputs must agree bit for bit; the
smaller calls are also checked against the fp64 oracle with the tolerances of
the parity tests (max |error| / RMS <= 2e-2 for bf16 inputs, 1e-4 for fp32)."""
import math

import numpy as np
import pytest
import torch

import gated_delta_rule_106_amd as kda
import oracle
from kda_workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

KEYS = ("q", "k", "v", "log_alpha", "beta", "gate")
DEV = "cuda:0"


def _err(got, ref):
    ref = np.asarray(ref)
    return float(np.abs(got.double().cpu().numpy() - ref).max()) / math.sqrt(float((ref ** 2).mean()))


def _both(wl, seed):
    x = make_inputs(wl, seed=seed)
    d = {k: (v.to(DEV) if v is not None else None) for k, v in x.items()}
    fin = wl.final_state
    print(f"[no-alloc] {wl.name} B{wl.B} H{wl.H} T{wl.T} d{wl.Dk} seed {seed}", flush=True)
    y0, s0 = kda.chunk_fwd(*(d[k] for k in KEYS), initial_state=d["initial_state"], output_final_state=fin,
                           chunk=wl.chunk)
    torch.cuda.synchronize()
    # outputs preallocated, no workspace: the call itself allocates nothing
    y1 = torch.full_like(y0, float("nan"))
    s1 = torch.full_like(s0, float("nan")) if fin else None
    kda.chunk_fwd(*(d[k] for k in KEYS), initial_state=d["initial_state"], output_final_state=fin,
                  chunk=wl.chunk, out=y1, final_state=s1, no_alloc=True)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    if fin:
        assert torch.equal(s0, s1)
    return x, y1, s1


def test_noalloc_matches_workspace_call_on_consecutive_calls():
    # call 1: the B1 H8 T4096 prefill, 512 cards in the fixed scratch
    _both(CONFIGS[1], seed=1)
    # call 2: smaller, ragged, with state in and out; its cards overwrite part of call 1's
    wl = CONFIGS[2].scaled(B=1, H=2, T=300, Dk=64, Dv=64)
    x, y, s = _both(wl, seed=21)
    yo, so = oracle.fwd(*(x[k] for k in KEYS), initial_state=x["initial_state"])
    assert _err(y, yo) <= 2e-2 and _err(s, so) <= 2e-2
    # call 3: smaller still, fp32 inputs on the chunk-16 path
    wl = CONFIGS[0].scaled(T=100)
    x, y, s = _both(wl, seed=22)
    yo, so = oracle.fwd(*(x[k] for k in KEYS))
    assert _err(y, yo) <= 1e-4 and _err(s, so) <= 1e-4
