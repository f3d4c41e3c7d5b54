"""The chunkwise backward's algebra (tests/_chunk_adjoint.py), chunk by chunk in fp64,
reproduces the oracle's token-by-token gradients and its forward: the formulas a
chunkwise GPU backward transcribes are exact, for any chunk size (page "Kimi K3
report walk-through", section "Hierarchical chunking of linear attention": the
chunk size does not change the result)."""
import numpy as np
import pytest

import oracle
from tests._chunk_adjoint import chunkwise_fwd_bwd

KEYS = ("q", "k", "v", "log_alpha", "beta", "gate")


@pytest.mark.parametrize("T,chunk,Dk,Dv", [(37, 8, 5, 4), (64, 16, 6, 3), (50, 64, 4, 4), (33, 1, 3, 2)])
def test_chunk_adjoint_matches_oracle_gradients(oracle_lib, T, chunk, Dk, Dv):
    rng = np.random.default_rng(900 + T + chunk)
    x = dict(q=rng.standard_normal((1, T, 1, Dk)) * 0.5, k=rng.standard_normal((1, T, 1, Dk)) * 0.5,
             v=rng.standard_normal((1, T, 1, Dv)), log_alpha=rng.uniform(-6.0, 0.3, (1, T, 1, Dk)),
             beta=rng.uniform(0.05, 0.95, (1, T, 1)), gate=rng.standard_normal((1, T, 1, Dv)))
    x = {n: a.astype(np.float32) for n, a in x.items()}  # some log alpha clamped on either side
    s0 = rng.standard_normal((1, 1, Dk, Dv)) * 0.4
    dy = rng.standard_normal((1, T, 1, Dv))
    dST = rng.standard_normal((1, 1, Dk, Dv))
    g = oracle.bwd(*(x[n] for n in KEYS), dy, initial_state=s0, d_final_state=dST)
    yo, so = oracle.fwd(*(x[n] for n in KEYS), initial_state=s0)
    y, sT, c = chunkwise_fwd_bwd(*(x[n][0, :, 0] for n in KEYS), dy[0, :, 0], s0[0, 0], dST[0, 0], chunk)
    rel = lambda a, b: np.abs(a - b).max() / max(np.abs(b).max(), 1e-30)
    assert rel(y, yo[0, :, 0]) <= 1e-10 and rel(sT, so[0, 0]) <= 1e-10
    for name in ("dq", "dk", "dv", "dlog_alpha", "dgate"):
        assert rel(c[name], g[name][0, :, 0]) <= 1e-9, name
    assert rel(c["dbeta"], g["dbeta"][0, :, 0]) <= 1e-9
    assert rel(c["dinitial_state"], g["dinitial_state"][0, 0]) <= 1e-9
