"""Seeded synthetic inputs for the KDA token mixer.

This module holds only input recipes: shapes, dtypes and value distributions.
It contains none of the method's arithmetic and is the single source of inputs
shared by the tests, the smoke check and the benchmark (both the HIP path and
the fp64 oracle consume exactly the tensors produced here).

Recipe (the pages give no activations; these stand in for them):
  q, k ~ N(0, 1), L2-normalised per (b, t, h) over the key dimension, and q then
  scaled by 1/sqrt(d_k); v ~ N(0, 1); beta = sigmoid(N(mu_beta, 1));
  log alpha per channel = max(logsigmoid(N(mu_alpha, 1)), ln 0.0067);
  gate logits ~ N(0, 1); optional fp32 initial state ~ N(0, 0.02^2).
The retention floor ln 0.0067 is the one stated on page "3T models are no
longer magic", section "Gate 1: KDA makes it computable" (about 0.67 % per
step).  Sampling happens in float32 on a CPU torch.Generator in the fixed order
q, k, v, beta, log alpha, gate, state; bfloat16 configurations are then cast
with round-to-nearest-even.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

LOG_ALPHA_FLOOR = math.log(0.0067)


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill" or "decode"
    B: int
    H: int
    T: int                    # tokens per sequence (1 for decode)
    Dk: int
    Dv: int
    dtype: str                # "f32" or "bf16": q, k, v, log alpha, beta, gate and output
    chunk: int = 64
    init_state: bool = False
    final_state: bool = False
    beta_mu: float = 0.0
    alpha_mu: float = 2.0
    floor_frac: float = 0.0   # fraction of key channels per head pinned at the floor
    seed: int = 0
    notes: str = field(default="", compare=False)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


CONFIGS = {
    0: Workload("kda_fwd_f32_B1_H2_T256_d64", "prefill", B=1, H=2, T=256, Dk=64, Dv=64,
                dtype="f32", chunk=16, final_state=True, seed=0,
                notes="fp32 correctness case, chunk 16, zero initial state"),
    1: Workload("kda_prefill_bf16_B1_H8_T4096_d128", "prefill", B=1, H=8, T=4096, Dk=128,
                Dv=128, dtype="bf16", chunk=64, seed=1,
                notes="chunk 64 built from 16-token sub-chunks, zero initial state"),
    2: Workload("kda_prefill_bf16_B2_H32_T8192_d128_state", "prefill", B=2, H=32, T=8192,
                Dk=128, Dv=128, dtype="bf16", chunk=64, init_state=True, final_state=True,
                seed=2, notes="random fp32 initial state, returns the final state"),
    3: Workload("kda_prefill_bf16_B1_H16_T65536_d128_floor", "prefill", B=1, H=16, T=65536,
                Dk=128, Dv=128, dtype="bf16", chunk=64, beta_mu=1.0, alpha_mu=3.0,
                floor_frac=0.3, seed=3,
                notes="30% of key channels per head at the retention floor every token"),
    4: Workload("kda_decode_bf16_B512_H32_d128", "decode", B=512, H=32, T=1, Dk=128, Dv=128,
                dtype="bf16", init_state=True, final_state=True, seed=4,
                notes="single-token step, fp32 128x128 state per head updated in place"),
}


def _normal(gen, shape, mu=0.0, std=1.0):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if mu != 0.0:
        x.add_(mu)
    return x


def make_inputs(wl: Workload, seed: int | None = None) -> dict:
    """Build the CPU tensors of one workload.

    Prefill: q, k, log_alpha [B, T, H, Dk]; v, gate [B, T, H, Dv]; beta [B, T, H];
    initial_state [B, H, Dk, Dv] float32 or None.
    Decode: the same without the T axis; ``state`` [B, H, Dk, Dv] float32.
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(wl.seed if seed is None else seed)
    B, H, T, Dk, Dv = wl.B, wl.H, wl.T, wl.Dk, wl.Dv
    lead = (B, H) if wl.kind == "decode" else (B, T, H)
    q = _normal(gen, lead + (Dk,))
    k = _normal(gen, lead + (Dk,))
    v = _normal(gen, lead + (Dv,))
    beta = torch.sigmoid(_normal(gen, lead, mu=wl.beta_mu))
    la = torch.nn.functional.logsigmoid(_normal(gen, lead + (Dk,), mu=wl.alpha_mu))
    la.clamp_(min=LOG_ALPHA_FLOOR)
    if wl.floor_frac > 0.0:
        n_floor = int(round(wl.floor_frac * Dk))
        # a fixed per-head subset of key channels sits at the floor for every token
        for h in range(H):
            perm = torch.randperm(Dk, generator=gen)[:n_floor]
            la[..., h, perm] = LOG_ALPHA_FLOOR
    gate = _normal(gen, lead + (Dv,))
    state = None
    if wl.init_state:
        state = _normal(gen, (B, H, Dk, Dv), std=0.02)
    # normalise q and k per token and head, scale q by 1/sqrt(d_k)
    q = q / q.norm(dim=-1, keepdim=True).clamp_min(1e-12) / math.sqrt(Dk)
    k = k / k.norm(dim=-1, keepdim=True).clamp_min(1e-12)
    dt = wl.torch_dtype
    out = dict(q=q.to(dt).contiguous(), k=k.to(dt).contiguous(), v=v.to(dt).contiguous(),
               log_alpha=la.to(dt).contiguous(), beta=beta.to(dt).contiguous(),
               gate=gate.to(dt).contiguous())
    if wl.kind == "decode":
        out["state"] = state if state is not None else torch.zeros(B, H, Dk, Dv)
    else:
        out["initial_state"] = state
    return out


def make_raw_inputs(wl: Workload, seed: int | None = None) -> dict:
    """Raw projections for the fused-preprocessing path: the same sampling as
    ``make_inputs`` up to, but not including, the per-token normalisation of q and
    k and the log-sigmoid of the forget logits.  Each token's q and k are also
    multiplied by a random factor in [0.1, 10) (projections come at any size).
    log_alpha holds the forget-gate logits x ~ N(mu_alpha, 1); channels pinned at
    the floor get x = -12 (log-sigmoid about -12, below ln 0.0067)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(wl.seed if seed is None else seed)
    B, H, T, Dk, Dv = wl.B, wl.H, wl.T, wl.Dk, wl.Dv
    lead = (B, H) if wl.kind == "decode" else (B, T, H)
    q = _normal(gen, lead + (Dk,))
    k = _normal(gen, lead + (Dk,))
    v = _normal(gen, lead + (Dv,))
    beta = torch.sigmoid(_normal(gen, lead, mu=wl.beta_mu))
    x = _normal(gen, lead + (Dk,), mu=wl.alpha_mu)
    if wl.floor_frac > 0.0:
        n_floor = int(round(wl.floor_frac * Dk))
        for h in range(H):
            perm = torch.randperm(Dk, generator=gen)[:n_floor]
            x[..., h, perm] = -12.0
    gate = _normal(gen, lead + (Dv,))
    state = _normal(gen, (B, H, Dk, Dv), std=0.02) if wl.init_state else None
    fq = torch.rand(lead + (1,), generator=gen) * 9.9 + 0.1
    fk = torch.rand(lead + (1,), generator=gen) * 9.9 + 0.1
    dt = wl.torch_dtype
    out = dict(q=(q * fq).to(dt).contiguous(), k=(k * fk).to(dt).contiguous(), v=v.to(dt).contiguous(),
               log_alpha=x.to(dt).contiguous(), beta=beta.to(dt).contiguous(),
               gate=gate.to(dt).contiguous())
    if wl.kind == "decode":
        out["state"] = state if state is not None else torch.zeros(B, H, Dk, Dv)
    else:
        out["initial_state"] = state
    return out


def small(wl: Workload, **kw) -> Workload:
    """A reduced copy of a workload (same recipe) for parity at oracle-friendly sizes."""
    return wl.scaled(**kw)
