#!/usr/bin/env python3
"""Throughput of the KDA token mixer on one MI355X (gfx950).

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one chunkwise prefill (cumulative log-decay, q/k rescaling, the
intra-chunk UT transform, the sequential state pass with the fused output read
and gate) over the largest single-GPU prefill workload: B=1, H=16, T=65536,
d_k = d_v = 128, bf16 inputs, fp32 state, chunk 64 built from 16-token tiles,
30 % of the key channels at the retention floor on every token.  The same run
times the other prefill shapes for context under ``configs`` (the fp32
correctness case, B1 H8 T4096, and B2 H32 T8192 with state in/out), each with
its own roofline object; the single-token decode step on B=512, H=32 (fp32
128x128 state per head, updated in place) in the ``decode`` object; ``varlen``
a mixed-length batch through the variable-length call (with and without state
snapshots) against padding it to one length; ``fused_prep`` B1 H8 T4096 on raw
q, k and forget logits with the preparation fused into the card builder;
``backward`` the gradient call on B1 H8 T4096; and ``context_parallel`` one
GPU's share of an 8-way split along T of the headline workload (segment
summary, ordered combination, re-run).

Algorithmic bytes count every input once and the output at the input dtype
(1538 B per head-token at d = 128 in bf16); the library writes an fp32 output,
whose extra 256 B per head-token are reported beside it
(``fp32_output_extra_bytes``), not folded into the fraction.

Inputs are synthetic and seeded (kda_workloads); they are resident in device
memory before the timed region starts.  Workloads smaller than the 256 MB
Infinity Cache rotate through several input sets whose total size exceeds it,
so their reads come from HBM.  Kernel durations come from HIP events recorded
on the stream the library launches on.  Rank 0 prints one JSON line on stdout;
progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s + % bf16 MFMA peak; decode steps/s + % HBM BW"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA, TFLOP/s
KEYS = ("q", "k", "v", "log_alpha", "beta", "gate")
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ----------------------------------------------------------- algorithmic work
def prefill_bytes(wl) -> int:
    """Algorithmic HBM bytes of one prefill: q, k, v, log alpha, gate and beta read
    once and y written once, all at the input dtype (2 B per element in bf16), plus
    one read of the initial and one write of the final fp32 state when present.
    At d = 128 in bf16: 1538 B per head-token."""
    esz = 2 if wl.dtype == "bf16" else 4
    per_tok = esz * (3 * wl.Dk + 3 * wl.Dv + 1)
    n = wl.B * wl.T * wl.H * per_tok
    st = wl.B * wl.H * wl.Dk * wl.Dv * 4
    return n + (st if wl.init_state else 0) + (st if wl.final_state else 0)


def fp32_output_extra_bytes(wl) -> int:
    """Bytes the fp32 output writes beyond an output at the input dtype (256 B per
    head-token at d = 128 with bf16 inputs; zero for fp32 inputs)."""
    esz = 2 if wl.dtype == "bf16" else 4
    return wl.B * wl.T * wl.H * wl.Dv * (4 - esz)


def prefill_flops(wl) -> int:
    """Algorithmic flops of the chunkwise form per head-token, causal triangles
    counted exactly: 2d[(C-1)/2 + 4(C+1)/2] + C^2/3 + 6 d^2 (A, P, W, U~ and
    P U triangles; the triangular solve; W S, Q~ S and Kbar^T U)."""
    C, d = wl.chunk, wl.Dk
    per = 2 * d * ((C - 1) / 2 + 4 * (C + 1) / 2) + C * C / 3 + 6 * d * d
    return int(round(per * wl.B * wl.T * wl.H))


def decode_bytes(wl) -> int:
    """Per (b, h): read and write of the fp32 state, q, k, v, log alpha, gate and
    beta read once and y written once at the input dtype (132 610 B at d = 128 in
    bf16)."""
    esz = 2 if wl.dtype == "bf16" else 4
    per = 2 * wl.Dk * wl.Dv * 4 + esz * (3 * wl.Dk + 3 * wl.Dv + 1)
    return wl.B * wl.H * per


def decode_flops(wl) -> int:
    return 7 * wl.Dk * wl.Dv * wl.B * wl.H


# ------------------------------------------------------------------ helpers
def source_digest() -> str:
    """Digest of the HIP sources, used to tell whether stored counter readings
    still describe the kernels being timed."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_106_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel_tag: str):
    """HBM bytes per launch from the committed counter summary, or None when it
    is absent or was taken on other kernel sources."""
    path = os.path.join(PROFILES, "traffic_" + kernel_tag + ".md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"^source_digest:\s*(\w+)", text, re.M)
    m_b = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m_src or not m_b or m_src.group(1) != source_digest():
        return None
    return float(m_b.group(1))


def stored_mfma_counters(tag: str):
    """MFMA utilisation (busy cycles over all SIMD cycles) and executed MFMA flops per
    call from the committed counter summary, or None when it is missing or was taken
    on other HIP sources."""
    path = os.path.join(PROFILES, "pmc_mfma_" + tag + ".md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"^source_digest:\s*(\w+)", text, re.M)
    m_u = re.search(r"^mfma_util_call:\s*([0-9.eE+-]+)", text, re.M)
    m_f = re.search(r"^mfma_executed_flops_per_call:\s*([0-9.eE+]+)", text, re.M)
    if not (m_src and m_u and m_f) or m_src.group(1) != source_digest():
        return None
    return {"mfma_util": float(m_u.group(1)), "executed_flops_per_call": float(m_f.group(1))}


def to_dev(x, dev):
    import torch
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def time_calls(fn, sets, steps, warmup, stream):
    """Run fn(set) W times untimed, then K times back to back between two
    synchronisations, with one HIP event pair on the launch stream around the
    K calls (an event between calls would itself cost GPU time).  Returns
    (wall seconds, event milliseconds per call)."""
    import torch
    for i in range(warmup):
        fn(sets[i % len(sets)])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        fn(sets[i % len(sets)])
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1) / steps


def prefill_sets(kda, wl, n_sets, dev, out_dtype=None):
    import torch
    from kda_workloads import make_inputs
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    sets = []
    ws_n = kda.workspace_bytes(wl.B, wl.T, wl.H, wl.Dk, dtype=wl.torch_dtype, chunk=wl.chunk)
    for i in range(n_sets):
        x = to_dev(make_inputs(wl, seed=wl.seed + 100 * i), dev)
        x["out"] = torch.empty((wl.B, wl.T, wl.H, wl.Dv), dtype=out_dtype, device=dev)
        x["ws"] = torch.empty(max(ws_n, 16), dtype=torch.uint8, device=dev)
        x["final"] = (torch.empty((wl.B, wl.H, wl.Dk, wl.Dv), dtype=torch.float32, device=dev)
                      if wl.final_state else None)
        sets.append(x)
    return sets


def prefill_call(kda, wl):
    def fn(x):
        kda.chunk_fwd(*(x[k] for k in KEYS), initial_state=x.get("initial_state"),
                      output_final_state=wl.final_state, chunk=wl.chunk, out=x["out"],
                      out_dtype=x["out"].dtype, final_state=x["final"], workspace=x["ws"])
    return fn


# ---------------------------------------------------------------- the legs
def prefill_kernel(wl) -> str:
    """The kernels one kda_chunk_fwd call of this workload launches.  Few long bf16
    sequences (at most 128 one-tile state-pass workgroups, at least 256 chunks) take
    the pipelined pieces (of 128 chunks from 512 chunks on, else of 64)."""
    if wl.dtype != "bf16":
        return "kda_chunk_fwd = kda_prep_kernel + kda_recur_kernel (one call, two launches)"
    nc = (wl.T + 63) // 64
    if wl.Dk == 128 and wl.B * wl.H * (wl.Dk // 16) <= 128 and nc >= 256:
        pl = 128 if nc >= 512 else 64
        n = (nc + pl - 1) // pl
        return (f"kda_chunk_fwd in {n} pieces of {pl} chunks = kda_prep64_kernel (piece 0's cards) + "
                f"{n - 1} x kda_piece64_kernel (state pass over piece i beside the card builder of piece "
                f"i + 1) + kda_rec64_kernel (last piece): one call, {n + 1} launches")
    return "kda_chunk_fwd = kda_prep64_kernel + kda_rec64_kernel (one call, two launches)"


def bench_prefill(kda, wl, steps, warmup, n_sets, dev, stream):
    log(f"prefill {wl.name}: building {n_sets} input set(s)")
    sets = prefill_sets(kda, wl, n_sets, dev)
    wall, ev_ms = time_calls(prefill_call(kda, wl), sets, steps, warmup, stream)
    toks = wl.B * wl.T
    nbytes, flops = prefill_bytes(wl), prefill_flops(wl)
    extra = fp32_output_extra_bytes(wl)
    res = {
        "workload": wl.name, "B": wl.B, "H": wl.H, "T": wl.T, "d": wl.Dk, "chunk": wl.chunk,
        "input_sets": n_sets, "ms_per_step_wall": 1e3 * wall / steps, "kernel_ms_mean": ev_ms,
        "tokens_per_s": toks / (wall / steps),
        "kernel_tokens_per_s": toks / (ev_ms / 1e3),
        "alg_bytes": nbytes, "fp32_output_extra_bytes": extra, "alg_flops": flops,
        "hbm_gbs": nbytes / (ev_ms / 1e3) / 1e9, "mfma_tflops": flops / (ev_ms / 1e3) / 1e12,
    }
    res["hbm_frac"] = res["hbm_gbs"] / HBM_PEAK_GBS
    res["mfma_frac"] = res["mfma_tflops"] / BF16_MFMA_PEAK_TFLOPS
    res["roofline"] = {
        "kernel": prefill_kernel(wl), "bound": "hbm", "achieved": res["hbm_gbs"],
        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": res["hbm_frac"],
        "traffic": stored_traffic("prefill_" + wl.name),
        "bytes_per_launch": nbytes, "launch_ms": ev_ms,
        "achieved_with_fp32_output": (nbytes + extra) / (ev_ms / 1e3) / 1e9,
    }
    res["mfma"] = {"achieved": res["mfma_tflops"], "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                   "frac": res["mfma_frac"], "alg_flops_per_step": flops,
                   "counters": stored_mfma_counters(wl.name)}
    log(f"prefill {wl.name}: {ev_ms * 1e3:.1f} us/call (events), "
        f"{res['tokens_per_s']:.3e} tok/s wall, {res['hbm_gbs']:.0f} GB/s alg "
        f"({100 * res['hbm_frac']:.1f} % of HBM peak), {100 * res['mfma_frac']:.2f} % MFMA alg")
    del sets
    return res, wall


def bench_bf16_output(kda, wl, steps, warmup, n_sets, dev, stream):
    """The same prefill call with y written in bf16 (the input dtype) instead of the
    default fp32: the bytes the call moves then equal the algorithmic count.  The
    default stays fp32 because rounding y to bf16 alone costs more than the 2e-2
    max-error-to-RMS budget on these outputs."""
    import torch
    sets = prefill_sets(kda, wl, n_sets, dev, out_dtype=torch.bfloat16)
    wall, ev_ms = time_calls(prefill_call(kda, wl), sets, steps, warmup, stream)
    del sets
    nbytes = prefill_bytes(wl)
    res = {"workload": wl.name, "out_dtype": "bf16", "input_sets": n_sets, "kernel_ms_mean": ev_ms,
           "tokens_per_s": wl.B * wl.T / (ev_ms / 1e3), "hbm_gbs": nbytes / (ev_ms / 1e3) / 1e9}
    res["hbm_frac"] = res["hbm_gbs"] / HBM_PEAK_GBS
    log(f"prefill {wl.name}, bf16 y: {ev_ms * 1e3:.1f} us/call (events), "
        f"{100 * res['hbm_frac']:.1f} % of HBM peak")
    return res


def bench_decode(kda, wl, steps, warmup, dev, stream):
    import torch
    from kda_workloads import make_inputs
    log(f"decode {wl.name}: building inputs")
    x = to_dev(make_inputs(wl), dev)
    x["out"] = torch.empty((wl.B, wl.H, wl.Dv), dtype=torch.float32, device=dev)
    state = x["state"]  # working copy, updated in place step after step

    def fn(_):
        kda.decode_step(*(x[k] for k in KEYS), state, out=x["out"])
    wall, ev_ms = time_calls(fn, [None], steps, warmup, stream)
    nbytes, flops = decode_bytes(wl), decode_flops(wl)
    extra = wl.B * wl.H * wl.Dv * (4 - (2 if wl.dtype == "bf16" else 4))
    res = {
        "workload": wl.name, "B": wl.B, "H": wl.H, "d": wl.Dk,
        "steps_per_s": 1e3 / ev_ms, "steps_per_s_wall": steps / wall,
        "tokens_per_s": wl.B * 1e3 / ev_ms, "kernel_ms_mean": ev_ms,
        "alg_bytes": nbytes, "fp32_output_extra_bytes": extra, "alg_flops": flops,
        "hbm_gbs": nbytes / (ev_ms / 1e3) / 1e9,
        "hbm_gbs_with_fp32_output": (nbytes + extra) / (ev_ms / 1e3) / 1e9,
    }
    res["hbm_frac"] = res["hbm_gbs"] / HBM_PEAK_GBS
    log(f"decode: {ev_ms * 1e3:.1f} us/step, {res['hbm_gbs']:.0f} GB/s "
        f"({100 * res['hbm_frac']:.1f} % of HBM peak)")
    return res


def _oracle_passes(oracle, wl, x, threads, budget_s, max_reps=1000):
    """Whole passes of the oracle over one workload until about budget_s seconds
    have been spent (at least one); returns (seconds per pass, passes)."""
    secs, reps = 0.0, 0
    while (secs < budget_s or reps == 0) and reps < max_reps:
        _, _, s = oracle.fwd(*(x[k] for k in KEYS), initial_state=x.get("initial_state"),
                             threads=threads, return_seconds=True)
        secs += s
        reps += 1
    return secs / reps, reps


def cpu_baseline(wl, budget_s, single_thread=()):
    """The fp64 oracle, as it stands, on the host cores: whole passes over the
    headline workload with OpenMP over (batch, head) until about budget_s seconds
    have been spent, plus one-thread times of the smaller workloads given."""
    import oracle
    from kda_workloads import make_inputs
    oracle.build(force=False)
    x = make_inputs(wl)
    threads = oracle.default_threads()
    used = max(1, min(threads, wl.B * wl.H))  # parallel over (batch, head) only
    per, reps = _oracle_passes(oracle, wl, x, threads, budget_s)
    log(f"cpu baseline: {per:.3f} s per pass over {wl.name} with {used} thread(s), {reps} pass(es)")
    res = {"value": wl.B * wl.T / per, "unit": "tokens/s", "cores": used, "kind": "oracle",
           "sample": f"{reps} whole pass(es) of the fp64 sequential oracle over {wl.name} "
                     f"(B={wl.B} H={wl.H} T={wl.T}); OpenMP over (batch, head), "
                     f"{threads} thread(s) available, {len(os.sched_getaffinity(0))} host core(s)",
           "seconds_per_pass": per}
    one = {}
    for w in single_thread:
        xs = make_inputs(w)
        per1, reps1 = _oracle_passes(oracle, w, xs, 1, min(2.0, budget_s / 4))
        one[w.name] = {"seconds_per_pass": per1, "passes": reps1, "tokens_per_s": w.B * w.T / per1,
                       "threads": 1}
        log(f"cpu baseline: {per1:.4f} s per pass over {w.name} on one thread, {reps1} pass(es)")
    if one:
        res["single_thread"] = one
    return res


def counter_pass(kda, head, dec_wl, n_sets, dev, stream):
    """A short run for hardware-counter collection (FETCH_SIZE, WRITE_SIZE, MFMA
    counters): a copy-shaped elementwise kernel of known size (1 GiB read, 1 GiB
    written) to calibrate the counters, then two calls of the headline prefill,
    the B1 H8 T4096 prefill once on each of n_sets rotating input sets, two calls
    of B2 H32 T8192 with state in/out, four decode steps and two backward calls
    on B1 H8 T4096.  The prefill dispatches of each workload are told apart by
    their grid sizes."""
    import torch
    from kda_workloads import CONFIGS
    n = 1 << 28
    src = torch.randn(n, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)  # reads 4n bytes, writes 4n bytes
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    timed = {}
    for wl, sets, calls in ((head, 1, 2), (CONFIGS[1], n_sets, n_sets), (CONFIGS[2], 1, 2)):
        pre, _ = bench_prefill(kda, wl, calls, 0, sets, dev, stream)
        timed[wl.name] = {"calls": calls, "input_sets": sets, "kernel_ms": pre["kernel_ms_mean"]}
        torch.cuda.empty_cache()
    dec = bench_decode(kda, dec_wl, 4, 0, dev, stream)
    # two backward calls on B1 H8 T4096
    from kda_workloads import make_inputs
    bw = CONFIGS[1]
    x = to_dev(make_inputs(bw, seed=bw.seed), dev)
    dy = torch.randn((bw.B, bw.T, bw.H, bw.Dv), generator=torch.Generator().manual_seed(bw.seed + 7))
    dy = dy.to(bw.torch_dtype).to(dev)
    ws = torch.empty(kda_bwd_workspace_bytes(bw), dtype=torch.uint8, device=dev)
    for _ in range(2):
        kda.chunk_bwd(*(x[k] for k in KEYS), dy, initial_state=x.get("initial_state"), workspace=ws,
                      need_initial_state_grad=False)
    torch.cuda.synchronize()
    return {"counter_pass": True, "backward_calls": 2, "backward_workload": bw.name,
            "calibration": {"kernel": "torch.neg fp32, 2^28 elements", "bytes_read": 4 * n,
                            "bytes_written": 4 * n},
            "prefill": timed, "decode_calls": 4, "decode_workload": dec_wl.name,
            "decode_kernel_ms": dec["kernel_ms_mean"], "source_digest": source_digest()}


def bench_context_parallel(kda, steps, warmup, dev, stream, P=8):
    """One GPU's share of a P-way split along T of the floor-stress workload (pages:
    "KDA context parallelism"): the summary of its T/P tokens, the ordered
    combination of the P summaries (P - 1 of which another GPU would deliver), and
    the re-run of its segment from the incoming state, on the cards the summary left
    (the re-run that builds them again is timed too).  Kernel time of each stage."""
    import torch
    from kda_workloads import CONFIGS, make_inputs
    full = CONFIGS[3]
    wl = full.scaled(T=full.T // P, init_state=True)
    log(f"context parallel: share of {P}-way split of {full.name}: T={wl.T} per GPU")
    x = to_dev(make_inputs(wl), dev)
    ws = torch.empty(kda.workspace_bytes(wl.B, wl.T, wl.H, wl.Dk), dtype=torch.uint8, device=dev)
    out = torch.empty((wl.B, wl.T, wl.H, wl.Dv), dtype=torch.float32, device=dev)
    M = torch.empty((wl.B, wl.H, wl.Dk, wl.Dk), dtype=torch.float32, device=dev)
    b = torch.empty((wl.B, wl.H, wl.Dk, wl.Dv), dtype=torch.float32, device=dev)
    kda.chunk_summary(x["k"], x["v"], x["log_alpha"], x["beta"], transition=M, offset=b, workspace=ws)
    Ms, bs = M.expand(P, *M.shape).contiguous(), b.expand(P, *b.shape).contiguous()
    fin = torch.empty_like(b)

    def f_sum(_):  # given q, it leaves complete cards for the re-run
        kda.chunk_summary(x["k"], x["v"], x["log_alpha"], x["beta"], transition=M, offset=b, workspace=ws,
                          q=x["q"])

    def f_comb(_):
        kda.combine_states(Ms, bs, x["initial_state"], segment_states=False, final_state=fin)

    def f_rerun_build(_):
        kda.chunk_fwd(*(x[k] for k in KEYS), initial_state=fin, out=out, workspace=ws)

    def f_rerun(_):  # the summary's cards, no card builder
        kda.chunk_fwd(*(x[k] for k in KEYS), initial_state=fin, out=out, workspace=ws, cards_ready=True)
    _, t_rb = time_calls(f_rerun_build, [None], steps, warmup, stream)
    _, t_sum = time_calls(f_sum, [None], steps, warmup, stream)
    _, t_comb = time_calls(f_comb, [None], steps, warmup, stream)
    _, t_rerun = time_calls(f_rerun, [None], steps, warmup, stream)
    units, d = wl.B * wl.H, wl.Dk
    # summary: reads k, v, log alpha (bf16) and beta; writes M and b (fp32)
    sum_bytes = wl.B * wl.T * wl.H * 2 * (2 * d + wl.Dv + 1) + units * 4 * d * (d + wl.Dv)
    # combination: per segment reads M_p and b_p, plus the initial and final state
    comb_bytes = units * 4 * d * (P * (d + wl.Dv) + 2 * wl.Dv)
    res = {"workload": full.name, "split": P, "tokens_per_gpu": wl.T, "B": wl.B, "H": wl.H, "d": d,
           "summary_us": 1e3 * t_sum, "combine_us": 1e3 * t_comb, "rerun_us": 1e3 * t_rerun,
           "rerun_building_cards_us": 1e3 * t_rb,
           "share_total_us": 1e3 * (t_sum + t_comb + t_rerun),
           "summary_alg_gbs": sum_bytes / (t_sum / 1e3) / 1e9,
           "combine_alg_gbs": comb_bytes / (t_comb / 1e3) / 1e9,
           "combine_tflops": units * P * 2 * d * d * wl.Dv / (t_comb / 1e3) / 1e12,
           "note": "per-GPU share only; the all-gather of the summaries between GPUs is not part "
                   "of this single-GPU measurement"}
    log(f"context parallel: summary {res['summary_us']:.1f} us, combine {res['combine_us']:.1f} us, "
        f"re-run {res['rerun_us']:.1f} us per GPU share")
    del x, ws, out
    torch.cuda.empty_cache()
    return res


def bench_fused_prep(kda, wl, steps, warmup, n_sets, dev, stream):
    """The headline prefill on raw projections with the preparation fused into the
    card builder (q/k L2 normalisation, log alpha from forget logits), against the
    same call on prepared inputs, and against preparing the raw inputs with separate
    torch ops before the plain call (the HBM round trip the fusion removes)."""
    import torch
    from kda_workloads import make_raw_inputs
    sets = prefill_sets(kda, wl, n_sets, dev)
    for i, x in enumerate(sets):  # same shapes; raw tensors in place of the prepared ones
        raw = to_dev(make_raw_inputs(wl, seed=wl.seed + 100 * i), dev)
        x.update({k: raw[k] for k in ("q", "k", "log_alpha")})

    def fused(x):
        kda.chunk_fwd(*(x[k] for k in KEYS), chunk=wl.chunk, out=x["out"], workspace=x["ws"],
                      qk_norm=True, gate_logits=True)

    def unfused(x):
        q, k = x["q"].float(), x["k"].float()
        qn = (q / q.norm(dim=-1, keepdim=True) / math.sqrt(wl.Dk)).to(x["q"].dtype)
        kn = (k / k.norm(dim=-1, keepdim=True)).to(x["k"].dtype)
        la = torch.nn.functional.logsigmoid(x["log_alpha"].float()).clamp_min(math.log(0.0067))
        kda.chunk_fwd(qn, kn, x["v"], la.to(x["log_alpha"].dtype), x["beta"], x["gate"], chunk=wl.chunk,
                      out=x["out"], workspace=x["ws"])
    _, t_f = time_calls(fused, sets, steps, warmup, stream)
    _, t_u = time_calls(unfused, sets, steps, warmup, stream)
    toks = wl.B * wl.T
    res = {"workload": wl.name, "fused_us": 1e3 * t_f, "host_prepared_then_plain_us": 1e3 * t_u,
           "fused_tokens_per_s": toks / (t_f / 1e3), "input_sets": n_sets,
           "fused_alg_gbs": prefill_bytes(wl) / (t_f / 1e3) / 1e9}
    log(f"fused preparation {wl.name}: {res['fused_us']:.1f} us/call fused, "
        f"{res['host_prepared_then_plain_us']:.1f} us with separate torch preparation")
    del sets
    torch.cuda.empty_cache()
    return res


def backward_bytes(wl) -> int:
    """Algorithmic HBM bytes of one backward call: the forward's inputs and d_out read
    once (bf16), the six fp32 gradients written once, plus the fp32 initial state and
    its gradient when present."""
    esz = 2 if wl.dtype == "bf16" else 4
    per_tok = wl.H * ((4 * wl.Dk + 2 * wl.Dv) * esz + esz + 4 * (3 * wl.Dk + 2 * wl.Dv) + 4)
    states = wl.B * wl.H * wl.Dk * wl.Dv * 4 * (2 if wl.init_state else 0)
    return wl.B * wl.T * per_tok + states


def kda_bwd_workspace_bytes(wl) -> int:
    """Workspace bytes of one kda_chunk_bwd call on this workload (host-side query)."""
    import ctypes
    from gated_delta_rule_106_amd import _abi
    a = _abi.BwdArgs()
    a.B, a.T, a.H, a.Dk, a.Dv = wl.B, wl.T, wl.H, wl.Dk, wl.Dv
    a.dtype = _abi.KDA_BF16 if wl.dtype == "bf16" else _abi.KDA_F32
    n = ctypes.c_size_t(0)
    rc = _abi.load().kda_chunk_bwd_workspace_size(ctypes.byref(a), ctypes.byref(n))
    if rc != 0:
        raise RuntimeError(f"kda_chunk_bwd_workspace_size: status {rc}")
    return max(int(n.value), 16)


def bench_backward(kda, wl, steps, warmup, dev, stream):
    """kda_chunk_bwd on the headline shape (gradients of sum(d_out * y) through the
    forward; fp32 arithmetic), timed like the forward."""
    import torch
    from kda_workloads import make_inputs
    x = to_dev(make_inputs(wl, seed=wl.seed), dev)
    g = torch.Generator(device="cpu").manual_seed(wl.seed + 7)
    x["dy"] = torch.randn((wl.B, wl.T, wl.H, wl.Dv), generator=g).to(wl.torch_dtype).to(dev)
    n_ws = kda_bwd_workspace_bytes(wl)
    x["bws"] = torch.empty(n_ws, dtype=torch.uint8, device=dev)

    def bwd(x):
        kda.chunk_bwd(*(x[k] for k in KEYS), x["dy"], initial_state=x.get("initial_state"),
                      workspace=x["bws"], need_initial_state_grad=False)
    _, t_b = time_calls(bwd, [x], steps, warmup, stream)
    toks = wl.B * wl.T
    byt = backward_bytes(wl)
    gbs = byt / (t_b / 1e3) / 1e9
    res = {"workload": wl.name, "us_per_call": 1e3 * t_b, "tokens_per_s": toks / (t_b / 1e3),
           "alg_bytes_per_call": byt, "alg_gbs": gbs, "workspace_bytes": n_ws,
           "compute": "fp32 (inputs bf16, gradients fp32)",
           "roofline": {"kernel": "kda_chunk_bwd = kda_bwd_chunk_kernel + kda_bwd_sweep_kernel + "
                                  "kda_bwd_grad_kernel (one call, three launches)",
                        "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS, "traffic": stored_traffic("backward_" + wl.name)}}
    log(f"backward {wl.name}: {res['us_per_call']:.1f} us/call, {res['tokens_per_s']:.3e} tok/s")
    del x
    torch.cuda.empty_cache()
    return res


def bench_varlen(kda, steps, warmup, dev, stream, N=32, H=8, snapshot_every=512):
    """A mixed-length batch (N sequences, lengths log-uniform in [64, 8192), seeded; the
    headline's distributions and head size) through the variable-length call, with and
    without state snapshots every snapshot_every tokens, against padding every sequence
    to the longest and running the batch call."""
    import torch
    from kda_workloads import CONFIGS, make_inputs
    g = torch.Generator().manual_seed(7)
    lengths = [int(64 * 2 ** (7 * float(u))) for u in torch.rand(N, generator=g)]
    rows, Tmax = sum(lengths), max(lengths)
    wl = CONFIGS[1].scaled(B=1, H=H, T=rows)
    x = {k: v[0] for k, v in to_dev(make_inputs(wl, seed=11), dev).items() if v is not None}
    cu = torch.tensor([0] + list(torch.tensor(lengths).cumsum(0)), dtype=torch.int64, device=dev)
    out = torch.empty((rows, H, wl.Dv), dtype=torch.float32, device=dev)
    pad = {k: torch.zeros((N, Tmax) + tuple(x[k].shape[1:]), dtype=x[k].dtype, device=dev) for k in KEYS}
    for i, L in enumerate(lengths):
        o = int(cu[i])
        for k in KEYS:
            pad[k][i, :L] = x[k][o:o + L]
    pws = torch.empty(kda.workspace_bytes(N, Tmax, H, wl.Dk), dtype=torch.uint8, device=dev)
    pout = torch.empty((N, Tmax, H, wl.Dv), dtype=torch.float32, device=dev)

    def var(_):
        kda.chunk_fwd_varlen(*(x[k] for k in KEYS), cu, out=out)

    def var_snap(_):
        kda.chunk_fwd_varlen(*(x[k] for k in KEYS), cu, out=out, snapshot_every=snapshot_every)

    def padded(_):
        kda.chunk_fwd(*(pad[k] for k in KEYS), out=pout, workspace=pws)
    _, t_v = time_calls(var, [None], steps, warmup, stream)
    _, t_s = time_calls(var_snap, [None], steps, warmup, stream)
    _, t_p = time_calls(padded, [None], steps, warmup, stream)
    res = {"sequences": N, "H": H, "d": wl.Dk, "tokens": rows, "longest": Tmax,
           "varlen_us": 1e3 * t_v, "varlen_snapshots_us": 1e3 * t_s, "snapshot_every": snapshot_every,
           "padded_batch_us": 1e3 * t_p, "varlen_tokens_per_s": rows / (t_v / 1e3),
           "note": "event time per call including the binding's allocations of outputs and workspace"}
    log(f"varlen: {N} sequences, {rows} tokens (longest {Tmax}): {res['varlen_us']:.1f} us, with snapshots every "
        f"{snapshot_every}: {res['varlen_snapshots_us']:.1f} us, padded batch {res['padded_batch_us']:.1f} us")
    del x, pad, pws, pout, out
    torch.cuda.empty_cache()
    return res


SEGMENT_SHAPES = ((1, 8, 4096), (1, 1, 16384), (1, 2, 32768), (1, 4, 16384), (2, 2, 8192))


def segment_sweep(kda, dev, stream, steps=20):
    """The segment scan against one sequential pass per (b, h), on few long
    sequences (bf16, d = 128, the headline's distributions): kernel time per call."""
    import torch
    from kda_workloads import CONFIGS, make_inputs
    rows = []
    for (B, H, T) in SEGMENT_SHAPES:
        wl = CONFIGS[1].scaled(B=B, H=H, T=T)
        x = to_dev(make_inputs(wl), dev)
        ws = torch.empty(kda.workspace_bytes(B, T, H, 128), dtype=torch.uint8, device=dev)
        out = torch.empty((B, T, H, 128), dtype=torch.float32, device=dev)
        r = {"B": B, "H": H, "T": T}
        for seg in (True, False):
            def fn(_):
                kda.chunk_fwd(*(x[k] for k in KEYS), out=out, workspace=ws, segment_scan=seg)
            _, ms = time_calls(fn, [None], steps, 3, stream)
            r["segments_us" if seg else "single_pass_us"] = 1e3 * ms
        log(f"segments B{B} H{H} T{T}: {r['segments_us']:.1f} us with, {r['single_pass_us']:.1f} us without")
        rows.append(r)
        del x, ws, out
        torch.cuda.empty_cache()
    return {"segment_sweep": rows, "source_digest": source_digest()}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sets", type=int, default=8, help="rotating prefill input sets")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="time budget of the oracle baseline (0 skips it)")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the context timings of the two larger prefill shapes")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the mixed-length batch (variable-length call, snapshots)")
    ap.add_argument("--no-fused-prep", action="store_true",
                    help="skip B1 H8 T4096 with the preparation fused in")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward pass on B1 H8 T4096")
    ap.add_argument("--no-bf16-output", action="store_true",
                    help="skip the headline prefill with y written in bf16")
    ap.add_argument("--no-context-parallel", action="store_true",
                    help="skip the per-GPU share of the context-parallel split")
    ap.add_argument("--segment-sweep", action="store_true",
                    help="time the segment scan against one pass per sequence on few long sequences")
    ap.add_argument("--counter-pass", action="store_true",
                    help="short run for rocprofv3 --pmc: counter calibration copy, the "
                         "headline prefill once per input set, four decode steps")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the KDA path here has no multi-GPU mode "
              "(its (batch, head) units shard with no communication; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_106_amd as kda
    from kda_workloads import CONFIGS

    kda._abi.load()  # raises if the HIP library is missing: there is no fallback
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    log(f"device {torch.cuda.get_device_name(dev)}; library {kda.library_path()}")

    head = CONFIGS[3]  # the largest single-GPU prefill workload
    if args.segment_sweep:
        print(json.dumps(segment_sweep(kda, dev, stream)), flush=True)
        return
    if args.counter_pass:
        print(json.dumps(counter_pass(kda, head, CONFIGS[4], args.sets, dev, stream)), flush=True)
        return
    # the headline's inputs (1.6 GB) are far beyond the Infinity Cache: one input set
    pre, wall = bench_prefill(kda, head, args.steps, args.warmup, 1, dev, stream)
    torch.cuda.empty_cache()
    if not args.no_bf16_output:
        pre["bf16_output"] = bench_bf16_output(kda, head, args.steps, args.warmup, 1, dev, stream)
        torch.cuda.empty_cache()
    dec = bench_decode(kda, CONFIGS[4], max(args.steps, 10), args.warmup, dev, stream)
    ctx = {}
    if not args.no_context:
        # B1 H8 T4096 (50 MB) rotates through args.sets input sets so that its reads come from HBM
        for cid, sets, steps in ((1, args.sets, args.steps), (2, 1, max(5, args.steps // 5)),
                                 (0, 1, max(5, args.steps // 5))):
            r, _ = bench_prefill(kda, CONFIGS[cid], steps, 2, sets, dev, stream)
            ctx[CONFIGS[cid].name] = r
            torch.cuda.empty_cache()
    small = CONFIGS[1]
    fprep = None
    if not args.no_fused_prep:
        fprep = bench_fused_prep(kda, small, args.steps, args.warmup, args.sets, dev, stream)
    vlen = None
    if not args.no_varlen:
        vlen = bench_varlen(kda, max(5, args.steps // 5), 2, dev, stream)
    bwd = None
    if not args.no_backward:
        bwd = bench_backward(kda, small, max(5, args.steps // 5), 2, dev, stream)
    kcp = None
    if not args.no_context_parallel:
        kcp = bench_context_parallel(kda, max(5, args.steps // 5), 2, dev, stream)

    out = {
        "metric": METRIC, "value": pre["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": pre["ms_per_step_wall"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "compute": "bf16 inputs; fp16/bf16 MFMA operands with fp32 accumulation; fp32 state; fp32 output",
        "data": "synthetic (seeded; q,k L2-normalised, q/sqrt(d), v~N(0,1), beta=sigmoid(N(1,1)), "
                "30% of key channels per head at log alpha = ln 0.0067 on every token, the rest "
                "max(logsigmoid(N(3,1)), ln 0.0067), gate~N(0,1))",
        "config": {"workload": head.name, "B": head.B, "H": head.H, "T": head.T, "d_k": head.Dk,
                   "d_v": head.Dv, "chunk": head.chunk, "global_batch": head.B,
                   "seq_len": head.T, "parallelism": "single GPU"},
        "mfma": pre["mfma"],
        "roofline": pre["roofline"],
        "decode": {"metric": "decode steps/s", "value": dec["steps_per_s"], "unit": "steps/s",
                   "tokens_per_s": dec["tokens_per_s"], "kernel_ms": dec["kernel_ms_mean"],
                   "roofline": {"kernel": "kda_decode_kernel", "bound": "hbm",
                                "achieved": dec["hbm_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": dec["hbm_frac"],
                                "traffic": stored_traffic("decode_" + CONFIGS[4].name),
                                "achieved_with_fp32_output": dec["hbm_gbs_with_fp32_output"]},
                   "workload": dec["workload"]},
        "prefill_detail": pre,
        "configs": ctx,
        "context_parallel": kcp,
        "fused_prep": fprep,
        "varlen": vlen,
        "backward": bwd,
        "source_digest": source_digest(),
    }
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(head, args.cpu_seconds, single_thread=(CONFIGS[0], CONFIGS[1]))
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
