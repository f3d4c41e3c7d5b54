"""The seeded input recipe: shapes, dtypes, determinism and distribution facts."""
import math

import torch

from kda_workloads import CONFIGS, LOG_ALPHA_FLOOR, make_inputs


def test_shapes_and_dtypes_small_copies():
    for cid, wl in CONFIGS.items():
        small = wl.scaled(B=min(wl.B, 2), H=min(wl.H, 3), T=min(wl.T, 40))
        x = make_inputs(small)
        lead = (small.B, small.H) if wl.kind == "decode" else (small.B, small.T, small.H)
        assert x["q"].shape == lead + (wl.Dk,)
        assert x["v"].shape == lead + (wl.Dv,)
        assert x["beta"].shape == lead
        assert x["q"].dtype == wl.torch_dtype
        if wl.kind == "decode":
            assert x["state"].shape == (small.B, small.H, wl.Dk, wl.Dv)
            assert x["state"].dtype == torch.float32
        elif wl.init_state:
            assert x["initial_state"].dtype == torch.float32


def test_deterministic_per_seed():
    wl = CONFIGS[1].scaled(T=64, H=2)
    a, b = make_inputs(wl), make_inputs(wl)
    for key in a:
        if a[key] is not None:
            assert torch.equal(a[key], b[key])
    c = make_inputs(wl, seed=99)
    assert not torch.equal(a["q"], c["q"])


def test_recipe_facts():
    wl = CONFIGS[0]
    x = make_inputs(wl)
    qn = x["q"].double().norm(dim=-1)
    kn = x["k"].double().norm(dim=-1)
    assert torch.allclose(qn, torch.full_like(qn, 1 / math.sqrt(wl.Dk)), rtol=1e-5)
    assert torch.allclose(kn, torch.ones_like(kn), rtol=1e-5)
    la = x["log_alpha"].double()
    assert la.max() < 0 and la.min() >= LOG_ALPHA_FLOOR - 1e-6
    b = x["beta"]
    assert 0 < b.min() and b.max() < 1


def test_floor_stress_fraction():
    wl = CONFIGS[3].scaled(T=32)
    x = make_inputs(wl)
    la = x["log_alpha"].float()  # bf16: the floor is exactly -5.0
    at_floor = (la == -5.0).all(dim=1)  # channel pinned for every token: [B, H, Dk]
    assert (at_floor.sum(dim=-1) >= round(0.3 * wl.Dk)).all()
