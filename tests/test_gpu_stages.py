"""The chunk-64 card builder's stages against their closed forms (the intermediate
quantities of the chunkwise form, page "Kimi K3 report walk-through", sections
"Compute paradigm" and "Hierarchical chunking of linear attention"), read back from
the workspace of a kda_chunk_fwd call through the C ABI.

For a chunk of C = 64 tokens with g the inclusive cumulative (clamped) log decay:
    Kt = k e^g,  Qt = q e^g,  Kbar = k e^{g_C - g},  Gamma = e^{g_C}
    A = strict_lower(diag(beta) Kt (k e^-g)^T),  P = lower(Qt (k e^-g)^T)
    T = (I + A)^-1 diag(beta)            (scipy.linalg.solve_triangular)
    W = T Kt,  U~ = T V,  Qe = Qt - P W,  Uo = P U~
computed here in fp64 with numpy from the same input bits.  The card keeps them as
fp16 MFMA fragments; the layout decoded below is the one the state pass reads (lane
l = 16 g + m, element j of a 16-byte fragment is channel 32 x + 4 g + (j mod 4) +
16 (j div 4) of K-step x).  Tolerance: 2e-3 of the block's largest magnitude (fp16
keeps 11 significant bits; the products take fp16 operands).
"""
import numpy as np
import pytest
import scipy.linalg
import torch

from kda_workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

C = 64
TOL = 2e-3
KEYS = ("q", "k", "v", "log_alpha", "beta", "gate")


def _card_layout(D):
    KB, NCT = D // 32, D // 16
    frag, hfrag = 1024, 512
    W = 0
    QE = W + 4 * KB * frag
    KBT = QE + 4 * KB * frag
    UT = KBT + NCT * 2 * frag
    UO = UT + NCT * 4 * hfrag
    GAM = UO + NCT * 4 * hfrag
    return dict(W=W, QE=QE, KBT=KBT, UT=UT, UO=UO, GAM=GAM, BYTES=GAM + D * 4)


def _decode(card, D):
    """One card's bytes -> (W, Qe, Kbar, U~, Uo, Gamma) as float64 arrays."""
    L = _card_layout(D)
    KB, NCT = D // 32, D // 16
    h16 = lambda off, n: np.frombuffer(card[off:off + 2 * n], dtype=np.float16).astype(np.float64)
    lanes = np.arange(64)
    g, m = lanes // 16, lanes % 16

    def rows_cm(base):  # [mt][kb] fragments of 64 lanes x 8 halves: X[16 mt + m][c(kb, g, j)]
        X = np.zeros((C, D))
        for mt in range(4):
            for kb in range(KB):
                f = h16(base + (mt * KB + kb) * 1024, 512).reshape(64, 8)
                for j in range(8):
                    ch = 32 * kb + 4 * g + (j & 3) + 16 * (j >> 2)
                    X[16 * mt + m, ch] = f[:, j]
        return X

    W = -rows_cm(L["W"])  # the card holds -W
    Qe = rows_cm(L["QE"])
    Kbar = np.zeros((C, D))  # pieces [ct][u][h] of 64 lanes x 4: Kbar[32 u + 16 h + 4 g + i][16 ct + m]
    for ct in range(NCT):
        for u in range(2):
            for hf in range(2):
                f = h16(L["KBT"] + ((ct * 2 + u) * 2 + hf) * 512, 256).reshape(64, 4)
                for i in range(4):
                    Kbar[32 * u + 16 * hf + 4 * g + i, 16 * ct + m] = f[:, i]

    def acc_blocks(base):  # [nt][mt] of 64 lanes x 4: X[16 mt + 4 g + i][16 nt + m]
        X = np.zeros((C, D))
        for nt in range(NCT):
            for mt in range(4):
                f = h16(base + (nt * 4 + mt) * 512, 256).reshape(64, 4)
                for i in range(4):
                    X[16 * mt + 4 * g + i, 16 * nt + m] = f[:, i]
        return X

    Ut = acc_blocks(L["UT"])
    Uo = acc_blocks(L["UO"])
    gam = np.frombuffer(card[L["GAM"]:L["GAM"] + 4 * D], dtype=np.float32).astype(np.float64)
    return W, Qe, Kbar, Ut, Uo, gam


def _closed_forms(x, b, h, n, D):
    """The chunk's stages in fp64 from the input bits (tokens past the end are identity
    steps: k = q = v = 0, beta = 0, log alpha = 0)."""
    T = x["q"].shape[1]
    rows = slice(n * C, min((n + 1) * C, T))
    L = rows.stop - rows.start
    pad = lambda a: np.concatenate([a, np.zeros((C - L,) + a.shape[1:])]) if L < C else a  # noqa: E731
    k = pad(x["k"][b, rows, h].double().numpy())
    q = pad(x["q"][b, rows, h].double().numpy())
    v = pad(x["v"][b, rows, h].double().numpy())
    la = pad(np.clip(x["log_alpha"][b, rows, h].double().numpy(), np.log(0.0067), 0.0))
    beta = pad(x["beta"][b, rows, h].double().numpy())
    g = np.cumsum(la, axis=0)
    E, gC = np.exp(g), g[-1]
    Kt, Qt, Kbar = k * E, q * E, k * np.exp(gC - g)
    Ki = k * np.exp(-g)  # fine in fp64 over one chunk
    A = np.tril(beta[:, None] * (Kt @ Ki.T), -1)
    P = np.tril(Qt @ Ki.T)
    Tm = scipy.linalg.solve_triangular(np.eye(C) + A, np.diag(beta), lower=True, unit_diagonal=True)
    W = Tm @ Kt
    Ut = Tm @ v
    return dict(W=W, Qe=Qt - P @ W, Kbar=Kbar, Ut=Ut, Uo=P @ Ut, gam=np.exp(gC))


def _rel(got, ref):
    return float(np.abs(got - ref).max()) / max(float(np.abs(ref).max()), 1e-30)


@pytest.mark.parametrize("D", [64, 128])
def test_card_stages_match_closed_forms(D):
    import gated_delta_rule_106_amd as kda
    wl = CONFIGS[3].scaled(B=2, H=2, T=100, Dk=D, Dv=D)  # 30 % of the channels at the floor
    x = make_inputs(wl, seed=91)
    d = {k: v.cuda() for k, v in x.items() if v is not None}
    nbytes = kda.workspace_bytes(wl.B, wl.T, wl.H, D)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    print(f"[stages] B{wl.B} H{wl.H} T{wl.T} D{D}", flush=True)
    kda.chunk_fwd(*(d[k] for k in KEYS), workspace=ws)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy().tobytes()
    CB = _card_layout(D)["BYTES"]
    NC = (wl.T + C - 1) // C
    worst = {}
    for b in range(wl.B):
        for h in range(wl.H):
            for n in range(NC):
                item = (b * wl.H + h) * NC + n
                W, Qe, Kbar, Ut, Uo, gam = _decode(raw[item * CB:(item + 1) * CB], D)
                ref = _closed_forms(x, b, h, n, D)
                for name, got in (("W", W), ("Qe", Qe), ("Kbar", Kbar), ("Ut", Ut), ("Uo", Uo), ("gam", gam)):
                    e = _rel(got, ref[name])
                    worst[name] = max(worst.get(name, 0.0), e)
    print("[stages] " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()), flush=True)
    for name, e in worst.items():
        assert e <= TOL, (name, e)
