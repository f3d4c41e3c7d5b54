"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch every one of them, while the real oracle passes.

Each mutant is a textual edit of ``oracle/kda_oracle.c`` compiled to a
temporary library; the pins are the brute-force expansion (tests/_brute.py),
the clamp semantics, the decode/prefill agreement and the explicit-matrix
segment summary.
"""
import numpy as np
import pytest

import oracle
from tests._brute import LOG_ALPHA_MIN, brute_fwd, brute_summary
from scipy.special import log_expit

MUTANTS = {
    "decay dropped": ("row[j] *= a;", "row[j] *= 1.0;"),
    "wrong sign in the correction": ("- r[j]);", "+ r[j]);"),
    "update strength dropped": ("u[j] = bt * (", "u[j] = ("),
    "read with the key instead of the query": ("o[j] += row[j] * qv[c];",
                                               "o[j] += row[j] * kv[c];"),
    "query reads the state before the write": ("o[j] += row[j] * qv[c];",
                                               "o[j] += (row[j] - kv[c] * u[j]) * qv[c];"),
    "transposed corrective write": ("row[j] += kv[c] * u[j];",
                                    "row[j] += kv[j % Dk] * u[c % Dv];"),
    "delta read before the forget": ("r[j] += row[j] * kv[c];",
                                     "r[j] += row[j] / exp(fmax(orc_load(la, dtype, tok * Dk + c),"
                                     " ORC_LOG_ALPHA_MIN)) * kv[c];"),
    "gate sign flipped": ("(1.0 + exp(-z))", "(1.0 + exp(z))"),
    "retention floor missing": ("if (l < ORC_LOG_ALPHA_MIN) l = ORC_LOG_ALPHA_MIN;", ""),
    "key of the previous token": ("kv[c] = orc_load(k, dtype, tok * Dk + c);",
                                  "kv[c] = orc_load(k, dtype, (t > 0 ? tok - H : tok) * Dk + c);"),
    # segment summary (transition product and zero-start state)
    "summary decay dropped": ("X[c * n + j] *= a[c];", "X[c * n + j] *= 1.0;"),
    "summary correction sign flipped": ("- bt * r[j];", "+ bt * r[j];"),
    "summary transposed write": ("X[c * n + j] += kv[c] * r[j];", "X[c * n + j] += kv[j % Dk] * r[c % n];"),
    "summary starts from zero instead of the identity": ("(i == j) ? 1.0 : 0.0", "0.0"),
    "summary value dropped": ("(vv ? bt * vv[j] : 0.0)", "0.0"),
    # fused preprocessing (raw q/k normalisation, forget-gate logits)
    "query scale dropped": ("orc_unit(kv, Dk, 1.0);\n            orc_unit(qv, Dk, sqrt((double)Dk));",
                            "orc_unit(kv, Dk, 1.0);\n            orc_unit(qv, Dk, 1.0);"),
    "key not normalised": ("orc_unit(kv, Dk, 1.0);", ""),
    "logsigmoid sign flipped": ("return x >= 0.0 ? -log1p(exp(-x))", "return x >= 0.0 ? log1p(exp(-x))"),
    "summary key not normalised": ("if (qk_norm) orc_unit(kk, Dk, 1.0);", ""),
}

# mistakes planted in the gradients (reverse mode); caught by differences of the forward
BWD_MUTANTS = {
    "backward: key-read term dropped": ("acc += G[c * Dv + j] * u[j] + Sh[c * Dv + j] * drv[j];",
                                        "acc += G[c * Dv + j] * u[j];"),
    "backward: decay missing on the state gradient": ("G[c * Dv + j] = a[c] * dsh;", "G[c * Dv + j] = dsh;"),
    "backward: gate derivative": ("dgate[tok * Dv + j] = g_y * o[j] * sg * (1.0 - sg);",
                                  "dgate[tok * Dv + j] = g_y * o[j] * sg;"),
    "backward: query gradient added after the write": ("G[c * Dv + j] += qv[c] * dov[j];",
                                                       "G[c * Dv + j] += 0.0 * qv[c] * dov[j];"),
    "backward: update strength dropped from dv": ("dv[tok * Dv + j] = bt * acc;", "dv[tok * Dv + j] = acc;"),
    "backward: log-sigmoid derivative dropped": ("(logits ? dl / (1.0 + exp(xg[c])) : dl)", "(logits ? dl : dl)"),
    "backward: normalisation's projection dropped": ("g[c] = (g[c] - raw[c] / nrm * dot) / (nrm * extra);",
                                                      "g[c] = g[c] / (nrm * extra);"),
}


def _bwd_pins_pass(handle) -> bool:
    """Gradients against central differences of the variant's own (unchanged) forward,
    on prepared inputs and on raw q, k and forget logits with the fused preparation."""
    rng = np.random.default_rng(78)
    B, T, H, Dk, Dv = 1, 3, 1, 2, 2
    keys = ("q", "k", "v", "log_alpha", "beta", "gate")
    cases = []
    x = dict(q=rng.standard_normal((B, T, H, Dk)) * 0.5, k=rng.standard_normal((B, T, H, Dk)) * 0.5,
             v=rng.standard_normal((B, T, H, Dv)), log_alpha=rng.uniform(-2, -0.1, (B, T, H, Dk)),
             beta=rng.uniform(0.1, 0.9, (B, T, H)), gate=rng.standard_normal((B, T, H, Dv)))
    cases.append(({k: a.astype(np.float32) for k, a in x.items()}, {}))
    xr = dict(x, q=x["q"] * 3.0, k=x["k"] * 0.4, log_alpha=rng.uniform(-3, 3, (B, T, H, Dk)))
    cases.append(({k: a.astype(np.float32) for k, a in xr.items()}, dict(qk_norm=True, gate_logits=True)))
    s0 = rng.standard_normal((B, H, Dk, Dv))
    dy = rng.standard_normal((B, T, H, Dv))
    for x, opts in cases:
        g = handle.bwd(*(x[n] for n in keys), dy, initial_state=s0, **opts)

        def loss(xx):
            y, _ = handle.fwd(*(xx[n] for n in keys), initial_state=s0, **opts)
            return float((y * dy).sum())
        h = np.float32(2.0 ** -10)
        for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("log_alpha", "dlog_alpha"),
                            ("beta", "dbeta"), ("gate", "dgate")):
            for idx in np.ndindex(x[name].shape):
                xp = {n: a.copy() for n, a in x.items()}
                xm = {n: a.copy() for n, a in x.items()}
                xp[name][idx] += h
                xm[name][idx] -= h
                fd = (loss(xp) - loss(xm)) / (2 * float(h))
                if abs(fd - g[gname][idx]) > 2e-5 * (1 + abs(fd)):
                    return False
    return True


def _pins_pass(handle) -> bool:
    rng = np.random.default_rng(77)
    B, T, H, Dk, Dv = 1, 6, 2, 4, 3
    q = (rng.standard_normal((B, T, H, Dk)) * 0.5).astype(np.float32)
    k = (rng.standard_normal((B, T, H, Dk)) * 0.5).astype(np.float32)
    v = rng.standard_normal((B, T, H, Dv)).astype(np.float32)
    la = rng.uniform(-8.0, 0.0, (B, T, H, Dk)).astype(np.float32)  # some below the floor
    beta = rng.uniform(0.1, 0.9, (B, T, H)).astype(np.float32)
    gate = rng.standard_normal((B, T, H, Dv)).astype(np.float32)
    s0 = rng.standard_normal((B, H, Dk, Dv))
    y, sT = handle.fwd(q, k, v, la, beta, gate, initial_state=s0)
    yb, sb = brute_fwd(q, k, v, la, beta, gate, s0=s0)
    if not (np.abs(y - yb).max() <= 1e-12 * np.abs(yb).max()
            and np.abs(sT - sb).max() <= 1e-12 * np.abs(sb).max()):
        return False
    M, bs = handle.summary(k, v, la, beta)
    Mb, bb = brute_summary(k, v, la, beta)
    if not (np.abs(M - Mb).max() <= 1e-12 * np.abs(Mb).max()
            and np.abs(bs - bb).max() <= 1e-12 * np.abs(bb).max()):
        return False
    # fused preprocessing: raw q, k of arbitrary size and forget logits
    qr = q * rng.uniform(0.1, 9, (B, T, H, 1)).astype(np.float32)
    kr = k * rng.uniform(0.1, 9, (B, T, H, 1)).astype(np.float32)
    x = (rng.standard_normal((B, T, H, Dk)) * 3).astype(np.float32)
    qn = qr.astype(np.float64) / np.linalg.norm(qr.astype(np.float64), axis=-1, keepdims=True) / np.sqrt(Dk)
    kn = kr.astype(np.float64) / np.linalg.norm(kr.astype(np.float64), axis=-1, keepdims=True)
    lx = np.maximum(log_expit(x.astype(np.float64)), LOG_ALPHA_MIN)
    y, sT = handle.fwd(qr, kr, v, x, beta, gate, initial_state=s0, qk_norm=True, gate_logits=True)
    yb, sb = brute_fwd(qn, kn, v, lx, beta, gate, s0=s0, clamp=False)
    if not (np.abs(y - yb).max() <= 1e-12 * np.abs(yb).max()
            and np.abs(sT - sb).max() <= 1e-12 * np.abs(sb).max()):
        return False
    M, bs = handle.summary(kr, v, x, beta, qk_norm=True, gate_logits=True)
    Mb, bb = brute_summary(kn, v, lx, beta, clamp=False)
    if not (np.abs(M - Mb).max() <= 1e-12 * np.abs(Mb).max()
            and np.abs(bs - bb).max() <= 1e-12 * np.abs(bb).max()):
        return False
    y1, s1 = handle.decode(*(np.ascontiguousarray(a[:, 0]) for a in (q, k, v, la, beta, gate)), s0)
    yb1, sb1 = brute_fwd(*(a[:, :1] for a in (q, k, v, la, beta, gate)), s0=s0)
    return bool(np.abs(y1 - yb1[:, 0]).max() <= 1e-12 * np.abs(yb1).max()
                and np.abs(s1 - sb1).max() <= 1e-12 * np.abs(sb1).max())


def test_real_oracle_passes_the_pins(oracle_lib):
    class _Real:
        fwd = staticmethod(oracle.fwd)
        decode = staticmethod(oracle.decode)
        summary = staticmethod(oracle.summary)
    assert _pins_pass(_Real())

    class _RealB:
        fwd = staticmethod(oracle.fwd)
        bwd = staticmethod(oracle.bwd)
    assert _bwd_pins_pass(_RealB())


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_planted_gradient_mistake_is_caught(tmp_path, name):
    old, new = BWD_MUTANTS[name]
    src = oracle.source_text()
    assert src.count(old) == 1, f"mutation anchor for '{name}' must occur exactly once"
    handle = oracle.compile_variant(src.replace(old, new), str(tmp_path / "mutant.so"))
    assert not _bwd_pins_pass(handle), f"gradient pins did not catch: {name}"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = oracle.source_text()
    assert src.count(old) == 1, f"mutation anchor for '{name}' must occur exactly once"
    handle = oracle.compile_variant(src.replace(old, new), str(tmp_path / "mutant.so"))
    assert not _pins_pass(handle), f"pins did not catch: {name}"
