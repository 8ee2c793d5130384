#!/usr/bin/env python3
"""Benchmark of the DeltaNet chunkwise forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--cp-groups G] [--gated]

One step = one call of ``deltanet_fwd`` (every kernel of the forward pass) over
one batch of synthetic inputs already resident in HBM. Every timed measurement
first runs its step untimed for ``SETTLE_S`` seconds so that the GPU clock
governor is in its steady state (a burst from idle dips for tens of ms), then
the W warmup steps, then exactly K timed steps between synchronisations. The default workload is
B=8, H=16, T=4096, dk=dv=128, chunk 64, bf16 (the paper-scale layer). Prints
one JSON line with the throughput (tokens/s), the fraction of the bf16
matrix-core peak, a roofline object for the dominant kernel (timed with HIP
events on the launch stream) and the fp64 CPU oracle's throughput on the
host cores. ``--gated`` measures Gated DeltaNet (``deltanet_gated_fwd``, with
per-token log decays) instead; without it, a short gated run of the same
workload is reported under ``variants.gated`` next to the headline figures.
``variants.bwd`` times ``deltanet_bwd`` (the backward pass: forward chain with
per-chunk states, reverse state-gradient chain, chunk-parallel finish) on the
same workload. ``variants.kda`` times ``deltanet_kda_fwd`` (per-channel decay) on the same
workload. ``variants.gdp`` times ``deltanet_gdp_fwd`` (Gated Delta Product, n_h = 2 substeps
per token) on the same B, H, T and widths. ``variants.kda_long`` and
``variants.gated_long`` time KDA and Gated DeltaNet on B=1 H=16 T=131072,
serial chain against context parallelism, and ``variants.bwd_long`` the
DeltaNet backward there (deltanet_bwd against deltanet_bwd_cp). ``variants.decode`` times ``deltanet_decode_step`` (one token per sequence and
head, state updated in place) on B=256 H=16 d=128 bf16, a 256 MiB state.
The other four workloads of the forward pass are timed by the same clock under
``variants.<workload>``: B=4 H=16 T=8192 (serial chain and the library's
context-parallel choice), B=1 H=16 T=131072 (serial chain against context
parallelism, with the speed-up), the packed batch of 64 sequences at H=32, and
the tiny fp32 case.

Accounting (per head-token, chunk C, key/value widths dk/dv):
  flops  F = 2C(3dk + 2dv) + 6 dk dv  -- the eight dense products of the
         per-chunk algorithm (KK^T, TK, TV, WS^T, QK^T, QS^T, PZ, Z^T K) as
         written, masked halves included; the T solve is not counted
  bytes  read q, k, v, beta (+ S0 when given), write o and S_final: the
         algorithmic minimum, each tensor touched once (gated: + g, fp32).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_FLOPS = 2.5e15   # MI355X dense bf16 matrix-core peak
PEAK_FP32_FLOPS = 157.3e12  # MI355X dense fp32 matrix-core peak
PEAK_HBM_BPS = 8.0e12      # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SRCS = [os.path.join(ROOT, "chunkwise_delta_rule_amd", "csrc", f)
               for f in ("chain_bf16.hip", "dn_work.h", "dn_internal.h")]


def flops_per_head_token(C, dk, dv):
    return 2 * C * (3 * dk + 2 * dv) + 6 * dk * dv


def flops_per_head_token_triangular(C, dk, dv):
    """The same eight products counting only the entries the masks keep:
    K K^T strictly lower ((C - 1) / 2C of the dense count), T K, T V, Q K^T
    and the masked scores times Z lower-inclusive ((C + 1) / 2C each); the
    three state products stay dense."""
    return (C - 1) * dk + (C + 1) * (2 * dk + 2 * dv) + 6 * dk * dv


def kernel_sha():
    """Hash of the sources of the dominant kernel (chain_kernel_ws); the
    committed counter summary is used only while it matches."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, esz, n_tokens, n_units, has_s0, has_sf, gated=False):
    per_tok = w.H * (2 * w.dk + 2 * w.dv + 1) * esz  # q, k, v, o, beta
    if gated:
        per_tok += w.H * 4  # g, fp32
    state = n_units * w.dv * w.dk * 4
    return n_tokens * per_tok + state * (int(has_s0) + int(has_sf))


# Untimed run of the step before its warmup, so that the clock governor is
# in its steady state when the timed region starts. On this part a burst of
# back-to-back launches first runs at the idle boost clock, then dips for
# about 30 ms (the layer forward goes from 141 to 180-205 us per launch) and
# settles near the boost figure; the settle phase covers the dip with margin.
SETTLE_S = 0.25


def settle(step, seconds=SETTLE_S):
    """Run ``step`` back to back, untimed, for about ``seconds`` of wall time
    (enqueued in batches, synchronised between batches). Returns the number
    of steps run."""
    import torch
    n, batch = 0, 1
    t_end = time.perf_counter() + seconds
    while True:
        for _ in range(batch):
            step()
        n += batch
        torch.cuda.synchronize()
        if time.perf_counter() >= t_end:
            return n
        batch = min(batch * 2, 256)


def time_steps(step, warmup, steps):
    """Settle (untimed, see ``settle``), run ``warmup`` untimed steps, then
    ``steps`` timed ones bracketed by synchronisations. Every launch goes on
    torch's current stream; one HIP event recorded there before the first
    timed step and one after the last bracket the region, so the steps run
    back to back with nothing between them. Returns (ms per step over the
    region, the same figure as the average launch duration of a one-launch
    step, wall seconds)."""
    import torch
    settle(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / steps
    return ms, ms, wall


def load_traffic(workload_name, gated=False):
    """HBM traffic from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source for this workload; else None."""
    path = os.path.join(PROFILES, f"traffic_chain{'_gated' if gated else ''}_{workload_name}.json")
    if not os.path.exists(path):
        return None
    try:
        t = json.load(open(path))
    except Exception:
        return None
    if t.get("kernel_source_sha") != kernel_sha() or t.get("workload") != workload_name:
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(inputs, w, varlen, budget_s, g=None):
    """Time the fp64 oracle on the host on a bounded sample of the workload
    (the gated oracle when log decays ``g`` are given)."""
    import numpy as np
    import torch
    import oracle

    def f64(t):
        return None if t is None else t.detach().to("cpu").to(torch.float64).numpy()

    threads = oracle.max_threads()
    if varlen:
        q, k, v, beta, cu, S0, lengths = inputs
        # sample: the first sequences (in index order) up to ~budget of work
        est_rate = 2.0e9 * threads  # flop/s, conservative
        n, work = 0, 0.0
        while n < len(lengths) and (work + lengths[n] * w.H * 6 * w.dk * w.dv) / est_rate < budget_s:
            work += lengths[n] * w.H * 6 * w.dk * w.dv
            n += 1
        n = max(n, 1)
        end = int(cu[n].item())
        args = [f64(x[:end]) for x in (q, k, v, beta)]
        cu_s = cu[:n + 1].cpu().numpy()
        t0 = time.perf_counter()
        if g is None:
            oracle.deltanet_fwd_varlen(*args, cu_s, None)
        else:
            oracle.gated_deltanet_fwd_varlen(*args, f64(g[:end]), cu_s, None)
        dt = time.perf_counter() - t0
        toks = end
        sample = f"first {n} of {len(lengths)} sequences ({toks} tokens x {w.H} heads)"
        units = n * w.H
    else:
        q, k, v, beta, S0 = inputs
        B = w.B
        est_rate = 2.0e9 * threads
        per_seq = w.T * w.H * 6 * w.dk * w.dv
        nb = max(1, min(B, int(budget_s * est_rate // per_seq)))
        args = [f64(x[:nb]) for x in (q, k, v, beta)]
        s0 = None if S0 is None else f64(S0[:nb])
        t0 = time.perf_counter()
        if g is None:
            oracle.deltanet_fwd(*args, s0)
        else:
            oracle.gated_deltanet_fwd(*args, f64(g[:nb]), s0)
        dt = time.perf_counter() - t0
        toks = nb * w.T
        sample = f"{nb} of {B} sequences ({toks} tokens x {w.H} heads)"
        units = nb * w.H
    return {"value": toks / dt, "unit": "tokens/s", "cores": int(min(threads, units)),
            "kind": "oracle", "sample": sample, "seconds": round(dt, 3), "cpu_model": cpu_model(),
            "host_threads": threads}


def bwd_variant(dev, w, inputs, fwd_ms, steps=10, warmup=3):
    """Time deltanet_bwd on the workload (dO ~ N(0, 1) in bf16, no final-state
    gradient). Bytes: the algorithmic minimum of reading q, k, v, beta, dO and
    writing dq, dk, dv, dbeta; the per-chunk states and partial sums the
    three passes exchange through HBM are reported separately."""
    import torch
    import chunkwise_delta_rule_amd as dn

    print("[bench] backward variant", file=sys.stderr, flush=True)
    q, k, v, beta, S0 = inputs
    g = torch.Generator(device=dev).manual_seed(9)
    dO = torch.randn(v.shape, generator=g, device=dev, dtype=torch.float32).to(v.dtype)
    need = dn.deltanet_bwd_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    ms, launch_ms, _ = time_steps(lambda: dn.deltanet_bwd(q, k, v, beta, dO, S0, workspace=ws), warmup, steps)
    esz = 2
    nbytes = w.B * w.T * w.H * (2 * (2 * w.dk + 2 * w.dv + 1)) * esz
    return {"call": "deltanet_bwd", "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 5),
            "tokens_per_s": round(w.B * w.T / (ms / 1e3), 1), "avg_launch_us": round(launch_ms * 1e3, 2),
            "vs_forward_time": round(launch_ms / fwd_ms, 3), "algorithmic_bytes": nbytes,
            "workspace_bytes": need, "hbm_frac_algorithmic": round(nbytes / (launch_ms / 1e3) / PEAK_HBM_BPS, 4)}


def gated_bwd_variant(dev, w, inputs, fwd_ms, steps=10, warmup=3):
    """Time deltanet_gated_bwd on the workload with the gated variant's log
    decays (synth.make_gates). Bytes: as bwd_variant plus g read and dg
    written (fp32, one per head-token)."""
    import torch
    import chunkwise_delta_rule_amd as dn
    from chunkwise_delta_rule_amd.synth import make_gates

    print("[bench] gated backward variant", file=sys.stderr, flush=True)
    q, k, v, beta, S0 = inputs
    gl = make_gates((w.B, w.T, w.H), seed=7, device=str(dev))
    g = torch.Generator(device=dev).manual_seed(9)
    dO = torch.randn(v.shape, generator=g, device=dev, dtype=torch.float32).to(v.dtype)
    need = dn.deltanet_gated_bwd_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    ms, launch_ms, _ = time_steps(lambda: dn.deltanet_gated_bwd(q, k, v, beta, gl, dO, S0, workspace=ws),
                                  warmup, steps)
    nbytes = w.B * w.T * w.H * (2 * (2 * (2 * w.dk + 2 * w.dv + 1)) + 2 * 4)
    return {"call": "deltanet_gated_bwd", "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 5),
            "tokens_per_s": round(w.B * w.T / (ms / 1e3), 1), "avg_launch_us": round(launch_ms * 1e3, 2),
            "vs_forward_time": round(launch_ms / fwd_ms, 3), "algorithmic_bytes": nbytes,
            "workspace_bytes": need, "hbm_frac_algorithmic": round(nbytes / (launch_ms / 1e3) / PEAK_HBM_BPS, 4)}


def kda_variant(dev, w, inputs, fwd_ms, steps=20, warmup=5):
    """Time deltanet_kda_fwd on the workload with per-channel log decays
    (synth.make_channel_gates). Bytes: q, k, v, beta, o plus g (fp32, dk per
    head-token)."""
    import torch
    import chunkwise_delta_rule_amd as dn
    from chunkwise_delta_rule_amd.synth import make_channel_gates

    print("[bench] kda variant", file=sys.stderr, flush=True)
    q, k, v, beta, S0 = inputs
    g = make_channel_gates((w.B, w.T, w.H, w.dk), seed=8, device=str(dev))
    o = torch.empty_like(v)
    Sf = torch.empty((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device=dev)
    ms, launch_ms, _ = time_steps(lambda: dn.deltanet_kda_fwd(q, k, v, beta, g, S0, o=o, S_final=Sf), warmup, steps)
    nbytes = w.B * w.T * w.H * (2 * (2 * w.dk + 2 * w.dv + 1) + 4 * w.dk) + w.B * w.H * w.dv * w.dk * 4
    return {"call": "deltanet_kda_fwd", "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 5),
            "tokens_per_s": round(w.B * w.T / (ms / 1e3), 1), "avg_launch_us": round(launch_ms * 1e3, 2),
            "vs_deltanet_time": round(launch_ms / fwd_ms, 3), "algorithmic_bytes": nbytes,
            "hbm_frac": round(nbytes / (launch_ms / 1e3) / PEAK_HBM_BPS, 4)}


def kda_long_variant(dev, B=1, H=16, T=131072, d=128, steps=5, warmup=2):
    """Time deltanet_kda_fwd on one long sequence per head (the long-context
    shape), serial chain against context parallelism at the library's group
    count; bytes as in kda_variant."""
    import torch
    import chunkwise_delta_rule_amd as dn
    from chunkwise_delta_rule_amd.synth import make_channel_gates, make_inputs

    print(f"[bench] kda long-context variant B={B} H={H} T={T}", file=sys.stderr, flush=True)
    q, k, v, beta, S0 = make_inputs(B, H, T, d, d, seed=11, device=str(dev))
    g = make_channel_gates((B, T, H, d), seed=11, device=str(dev))
    o = torch.empty_like(v)
    Sf = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    G = 0  # the KDA forward's own choice of group count (the workspace query's covers it)
    ws = torch.empty(max(dn.deltanet_workspace_bytes(B, H, T, d, d, 64, G), 1), dtype=torch.uint8, device=dev)
    out = {"call": "deltanet_kda_fwd", "config": {"B": B, "H": H, "T": T, "dk": d, "dv": d}, "steps": steps,
           "warmup": warmup}
    nbytes = B * T * H * (2 * (4 * d + 1) + 4 * d) + B * H * d * d * 4
    for name, groups in (("serial", 1), ("context_parallel", G)):
        ms, _, _ = time_steps(lambda: dn.deltanet_kda_fwd(q, k, v, beta, g, S0, o=o, S_final=Sf,
                                                          cp_groups=groups, workspace=ws), warmup, steps)
        out[name] = {"cp_groups": groups, "ms_per_step": round(ms, 4),
                     "tokens_per_s": round(B * T / (ms / 1e3), 1),
                     "hbm_frac": round(nbytes / (ms / 1e3) / PEAK_HBM_BPS, 4)}
    out["speedup"] = round(out["serial"]["ms_per_step"] / out["context_parallel"]["ms_per_step"], 3)
    return out


def bwd_long_variant(dev, B=1, H=16, T=131072, d=128, steps=3, warmup=1):
    """Time deltanet_bwd and deltanet_gated_bwd on one long sequence per head
    (the long-context shape), serial chains against context parallelism at
    the library's group count (deltanet_bwd_cp, deltanet_gated_bwd_cp); bytes
    as in bwd_variant."""
    import torch
    import chunkwise_delta_rule_amd as dn
    from chunkwise_delta_rule_amd.synth import make_inputs

    print(f"[bench] backward long-context variant B={B} H={H} T={T}", file=sys.stderr, flush=True)
    q, k, v, beta, S0 = make_inputs(B, H, T, d, d, seed=13, device=str(dev))
    g = torch.Generator(device=dev).manual_seed(14)
    dO = torch.randn(v.shape, generator=g, device=dev, dtype=torch.float32).to(v.dtype)
    G = 0  # the backward's own choice of group count
    ws = torch.empty(max(dn.deltanet_bwd_cp_workspace_bytes(B, H, T, d, d, 64, G), 1), dtype=torch.uint8,
                     device=dev)
    out = {"call": "deltanet_bwd / deltanet_bwd_cp (gated_*: deltanet_gated_bwd / deltanet_gated_bwd_cp)", "config": {"B": B, "H": H, "T": T, "dk": d, "dv": d},
           "steps": steps, "warmup": warmup}
    nbytes = B * T * H * 2 * (2 * (2 * d + 2 * d + 1))  # read q, k, v, beta, dO; write dq, dk, dv, dbeta
    for name, groups in (("serial", 1), ("context_parallel", G)):
        ms, _, _ = time_steps(lambda: dn.deltanet_bwd(q, k, v, beta, dO, S0, cp_groups=groups, workspace=ws),
                              warmup, steps)
        out[name] = {"cp_groups": groups, "ms_per_step": round(ms, 4),
                     "tokens_per_s": round(B * T / (ms / 1e3), 1),
                     "hbm_frac_algorithmic": round(nbytes / (ms / 1e3) / PEAK_HBM_BPS, 4)}
    out["speedup"] = round(out["serial"]["ms_per_step"] / out["context_parallel"]["ms_per_step"], 3)
    # the same for the Gated DeltaNet backward (deltanet_gated_bwd / deltanet_gated_bwd_cp)
    from chunkwise_delta_rule_amd.synth import make_gates
    gl = make_gates((B, T, H), seed=13, device=str(dev))
    del ws
    ws = torch.empty(max(dn.deltanet_gated_bwd_cp_workspace_bytes(B, H, T, d, d, 64, G), 1), dtype=torch.uint8,
                     device=dev)
    gbytes = nbytes + B * T * H * 8  # g read, dg written (fp32)
    for name, groups in (("gated_serial", 1), ("gated_context_parallel", G)):
        ms, _, _ = time_steps(lambda: dn.deltanet_gated_bwd(q, k, v, beta, gl, dO, S0, cp_groups=groups,
                                                            workspace=ws), warmup, steps)
        out[name] = {"cp_groups": groups, "ms_per_step": round(ms, 4),
                     "tokens_per_s": round(B * T / (ms / 1e3), 1),
                     "hbm_frac_algorithmic": round(gbytes / (ms / 1e3) / PEAK_HBM_BPS, 4)}
    out["gated_speedup"] = round(out["gated_serial"]["ms_per_step"] / out["gated_context_parallel"]["ms_per_step"], 3)
    del q, k, v, beta, dO, gl, ws
    torch.cuda.empty_cache()
    return out


def gated_long_variant(dev, B=1, H=16, T=131072, d=128, steps=5, warmup=2):
    """Time deltanet_gated_fwd on one long sequence per head (the long-context
    shape), serial chain against context parallelism at the library's group
    count; bytes: q, k, v, beta, o in bf16 and g in fp32 per head-token."""
    import torch
    import chunkwise_delta_rule_amd as dn
    from chunkwise_delta_rule_amd.synth import make_gates, make_inputs

    print(f"[bench] gated long-context variant B={B} H={H} T={T}", file=sys.stderr, flush=True)
    q, k, v, beta, S0 = make_inputs(B, H, T, d, d, seed=12, device=str(dev))
    g = make_gates((B, T, H), seed=12, device=str(dev))
    o = torch.empty_like(v)
    Sf = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    G = dn.deltanet_pick_cp_groups(B, H, T, d, d, 64)
    ws = torch.empty(max(dn.deltanet_workspace_bytes(B, H, T, d, d, 64, G), 1), dtype=torch.uint8, device=dev)
    out = {"call": "deltanet_gated_fwd", "config": {"B": B, "H": H, "T": T, "dk": d, "dv": d}, "steps": steps,
           "warmup": warmup}
    nbytes = B * T * H * (2 * (4 * d + 1) + 4) + B * H * d * d * 4
    for name, groups in (("serial", 1), ("context_parallel", G)):
        ms, _, _ = time_steps(lambda: dn.deltanet_gated_fwd(q, k, v, beta, g, S0, o=o, S_final=Sf,
                                                            cp_groups=groups, workspace=ws), warmup, steps)
        out[name] = {"cp_groups": groups, "ms_per_step": round(ms, 4),
                     "tokens_per_s": round(B * T / (ms / 1e3), 1),
                     "hbm_frac": round(nbytes / (ms / 1e3) / PEAK_HBM_BPS, 4)}
    out["speedup"] = round(out["serial"]["ms_per_step"] / out["context_parallel"]["ms_per_step"], 3)
    return out


def gdp_variant(dev, w, flops_per_head_step, peak_flops, nh=2, steps=20, warmup=5):
    """Time deltanet_gdp_fwd with nh substeps per token on the workload's B, H,
    T (real tokens) and widths: the chunkwise path runs over T nh virtual
    steps. Bytes: q, g, o per real token; k, v, beta per substep."""
    import torch
    import chunkwise_delta_rule_amd as dn
    from chunkwise_delta_rule_amd.synth import make_gates, make_inputs

    print(f"[bench] gdp variant n_h={nh}", file=sys.stderr, flush=True)
    B, H, T = w.B, w.H, w.T
    q, _, _, _, _ = make_inputs(B, H, T, w.dk, w.dv, seed=6, device=str(dev))
    _, k, v, beta, _ = make_inputs(B, H, T * nh, w.dk, w.dv, seed=7, device=str(dev))
    k, v, beta = k.view(B, T, nh, H, w.dk), v.view(B, T, nh, H, w.dv), beta.view(B, T, nh, H)
    g = make_gates((B, T, H), seed=6, device=str(dev))
    o = torch.empty((B, T, H, w.dv), dtype=q.dtype, device=dev)
    Sf = torch.empty((B, H, w.dv, w.dk), dtype=torch.float32, device=dev)
    ms, launch_ms, _ = time_steps(lambda: dn.deltanet_gdp_fwd(q, k, v, beta, g, None, o=o, S_final=Sf),
                                  warmup, steps)
    nbytes = B * T * H * (2 * (w.dk + w.dv) + 4 + nh * 2 * (w.dk + w.dv + 1)) + B * H * w.dv * w.dk * 4
    flops = B * T * nh * H * flops_per_head_step
    return {"call": "deltanet_gdp_fwd", "n_h": nh, "steps": steps, "warmup": warmup,
            "ms_per_step": round(ms, 5), "tokens_per_s": round(B * T / (ms / 1e3), 1),
            "virtual_steps_per_s": round(B * T * nh / (ms / 1e3), 1),
            "avg_launch_us": round(launch_ms * 1e3, 2), "algorithmic_bytes": nbytes,
            "hbm_frac": round(nbytes / (launch_ms / 1e3) / PEAK_HBM_BPS, 4),
            "mfma_frac": round(flops / (launch_ms / 1e3) / peak_flops, 4)}


def gdp_bwd_variant(dev, w, fwd_ms, nh=2, steps=10, warmup=3):
    """Time deltanet_gdp_bwd with nh substeps per token on the workload's B, H,
    T (real tokens), inputs drawn as in gdp_variant. Bytes: q, g, dO, dq, dg
    per real token; k, v, beta, dk, dv, dbeta per substep."""
    import torch
    import chunkwise_delta_rule_amd as dn
    from chunkwise_delta_rule_amd.synth import make_gates, make_inputs

    print(f"[bench] gdp backward variant n_h={nh}", file=sys.stderr, flush=True)
    B, H, T = w.B, w.H, w.T
    q, _, _, _, _ = make_inputs(B, H, T, w.dk, w.dv, seed=6, device=str(dev))
    _, k, v, beta, _ = make_inputs(B, H, T * nh, w.dk, w.dv, seed=7, device=str(dev))
    k, v, beta = k.view(B, T, nh, H, w.dk), v.view(B, T, nh, H, w.dv), beta.view(B, T, nh, H)
    g = make_gates((B, T, H), seed=6, device=str(dev))
    gen = torch.Generator(device=dev).manual_seed(9)
    dO = torch.randn((B, T, H, w.dv), generator=gen, device=dev, dtype=torch.float32).to(q.dtype)
    need = dn.deltanet_gdp_bwd_workspace_bytes(B, H, T, nh, w.dk, w.dv)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    ms, launch_ms, _ = time_steps(lambda: dn.deltanet_gdp_bwd(q, k, v, beta, g, dO, workspace=ws), warmup, steps)
    nbytes = B * T * H * 2 * (2 * (w.dk + w.dv) + 4 + nh * 2 * (w.dk + w.dv + 1))
    return {"call": "deltanet_gdp_bwd", "n_h": nh, "steps": steps, "warmup": warmup,
            "ms_per_step": round(ms, 5), "tokens_per_s": round(B * T / (ms / 1e3), 1),
            "virtual_steps_per_s": round(B * T * nh / (ms / 1e3), 1),
            "avg_launch_us": round(launch_ms * 1e3, 2), "vs_forward_time": round(launch_ms / fwd_ms, 3),
            "algorithmic_bytes": nbytes, "workspace_bytes": need,
            "hbm_frac_algorithmic": round(nbytes / (launch_ms / 1e3) / PEAK_HBM_BPS, 4)}


def metric_for(w):
    """The metric string with the workload's own shape in it."""
    if w.varlen:
        shape = f"N={w.N} packed L~U[{w.len_lo},{w.len_hi}] H={w.H} d={w.dk}"
    else:
        shape = f"B={w.B} H={w.H} T={w.T} d={w.dk}"
    prec = "bf16" if w.dtype == "bf16" else "fp32"
    return f"forward tokens/sec + % {prec} MFMA peak, {shape} chunk={w.chunk}"


def workload_variant(dev, name, cp_list=(1,), steps=10, warmup=3, seed=2):
    """Time deltanet_fwd (or deltanet_fwd_varlen) on another of the five
    workloads, once per entry of ``cp_list`` (1 serial chunk chain, 0 the
    library's group count, G > 1 forced). Bytes and flops as for the headline
    line. With a serial and an automatic entry the ratio of their times is
    reported as ``cp_speedup``."""
    import torch
    import chunkwise_delta_rule_amd as dn
    from chunkwise_delta_rule_amd.synth import WORKLOADS, workload_inputs

    w = WORKLOADS[name]
    print(f"[bench] workload variant {name}", file=sys.stderr, flush=True)
    inputs = workload_inputs(w, seed=seed, device=str(dev))
    esz = 2 if w.dtype == "bf16" else 4
    peak = PEAK_BF16_FLOPS if w.dtype == "bf16" else PEAK_FP32_FLOPS
    out = {"metric": metric_for(w), "steps": steps, "warmup": warmup}
    if w.varlen:
        q, k, v, beta, cu, S0, lengths = inputs
        n_tokens, n_units = int(sum(lengths)), w.N * w.H
        order = dn.longest_first_order(cu)
        o = torch.empty_like(v)
        Sf = torch.empty((w.N, w.H, w.dv, w.dk), dtype=torch.float32, device=dev)
        runs = [("serial", 1, lambda: dn.deltanet_fwd_varlen(q, k, v, beta, cu, S0, seq_order=order, o=o,
                                                             S_final=Sf))]
        out["config"] = {"N": w.N, "H": w.H, "total_T": n_tokens, "dk": w.dk, "dv": w.dv, "chunk": w.chunk}
    else:
        q, k, v, beta, S0 = inputs
        n_tokens, n_units = w.B * w.T, w.B * w.H
        o = torch.empty_like(v)
        Sf = torch.empty((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device=dev)
        runs = []
        for cp in cp_list:
            G = cp if cp > 0 else dn.deltanet_pick_cp_groups(w.B, w.H, w.T, w.dk, w.dv, w.chunk)
            ws = torch.empty(max(dn.deltanet_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, w.chunk, G), 1),
                             dtype=torch.uint8, device=dev)
            label = "serial" if G == 1 and cp == 1 else ("context_parallel_auto" if cp == 0 else f"cp{G}")
            runs.append((label, G, lambda G=G, ws=ws: dn.deltanet_fwd(q, k, v, beta, S0, o=o, S_final=Sf,
                                                                      cp_groups=G, workspace=ws)))
        out["config"] = {"B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv, "chunk": w.chunk}
    nbytes = algorithmic_bytes(w, esz, n_tokens, n_units, S0 is not None, True)
    flops = n_tokens * w.H * flops_per_head_token(w.chunk, w.dk, w.dv)
    out["algorithmic_bytes"] = nbytes
    out["flops_per_step"] = flops
    for label, G, fn in runs:
        ms, launch_ms, _ = time_steps(fn, warmup, steps)
        out[label] = {"cp_groups": G, "ms_per_step": round(ms, 5), "tokens_per_s": round(n_tokens / (ms / 1e3), 1),
                      "hbm_frac": round(nbytes / (ms / 1e3) / PEAK_HBM_BPS, 4),
                      "mfma_frac": round(flops / (ms / 1e3) / peak, 4)}
    if "serial" in out and "context_parallel_auto" in out:
        out["cp_speedup"] = round(out["serial"]["ms_per_step"] / out["context_parallel_auto"]["ms_per_step"], 3)
    if not bool(torch.isfinite(o).all()) or not bool(torch.isfinite(Sf).all()):
        print(f"bench.py: non-finite output in workload variant {name}", file=sys.stderr)
        sys.exit(3)
    del inputs, q, k, v, beta, o, Sf
    torch.cuda.empty_cache()
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def decode_variant(dev, B=256, H=16, d=128, steps=50, warmup=10):
    """Time deltanet_decode_step (with and without decay) and
    deltanet_kda_decode_step (per-channel decay) on a B x H state of d x d
    fp32 in place; bytes = the state read and written plus the token's
    vectors (q, k, v, o, beta, g)."""
    import torch
    import chunkwise_delta_rule_amd as dn
    from chunkwise_delta_rule_amd.synth import make_gates, make_inputs

    print(f"[bench] decode variant B={B} H={H} d={d}", file=sys.stderr, flush=True)
    q, k, v, beta, S = make_inputs(B, H, 1, d, d, seed=5, device=str(dev), s0_std=0.1)
    q, k, v, beta = (x[:, 0].contiguous() for x in (q, k, v, beta))
    g = make_gates((B, H), seed=5, device=str(dev))
    o = torch.empty_like(v)
    out = {"call": "deltanet_decode_step", "config": {"B": B, "H": H, "dk": d, "dv": d, "dtype": "bf16"},
           "steps": steps, "warmup": warmup}
    from chunkwise_delta_rule_amd.synth import make_channel_gates
    gk = make_channel_gates((B, 1, H, d), seed=5, device=str(dev))[:, 0].contiguous()
    for name, gg in (("plain", None), ("gated", g), ("kda", gk)):
        if name == "kda":
            step = lambda: dn.deltanet_kda_decode_step(q, k, v, beta, S, gk, o=o)
        else:
            step = lambda: dn.deltanet_decode_step(q, k, v, beta, S, gg, o=o)
        ms, launch_ms, _ = time_steps(step, warmup, steps)
        nbytes = B * H * (2 * d * d * 4 + 2 * (2 * d + 2 * d + 1) + (0 if gg is None else 4 * gg[0, 0].numel()))
        out[name] = {"ms_per_step": round(ms, 5), "avg_launch_us": round(launch_ms * 1e3, 2),
                     "tokens_per_s": round(B / (ms / 1e3), 1), "algorithmic_bytes": nbytes,
                     "achieved_GBps": round(nbytes / (launch_ms / 1e3) / 1e9, 1),
                     "hbm_frac": round(nbytes / (launch_ms / 1e3) / PEAK_HBM_BPS, 4)}
    if not bool(torch.isfinite(S).all()):
        print("bench.py: non-finite decode state", file=sys.stderr)
        sys.exit(3)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="layer_b8_h16_t4096")
    ap.add_argument("--cp-groups", type=int, default=1,
                    help="1 serial chunk chain, 0 library choice, G>1 forced")
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="target seconds of oracle work for the CPU baseline sample")
    ap.add_argument("--gated", action="store_true",
                    help="measure Gated DeltaNet (per-token log decays) instead of DeltaNet")
    ap.add_argument("--variants", default="all",
                    help="comma-separated variants to run after the main line (gated, bwd, gated_bwd, gdp, gdp_bwd, "
                         "kda, kda_long, gated_long, bwd_long, workloads, decode), or all")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the short gated and decode runs reported under variants")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain device copy of 1 GiB (for counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only; --gpus {args.gpus} is not supported "
              "(how the path would shard across GPUs is described in the design notes, not implemented).", file=sys.stderr)
        sys.exit(2)

    import torch
    import chunkwise_delta_rule_amd as dn
    from chunkwise_delta_rule_amd.synth import WORKLOADS, make_gates, workload_inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WORKLOADS[args.workload]
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    esz = 2 if w.dtype == "bf16" else 4

    print(f"[bench] workload {w.name}: generating inputs on {dev}", file=sys.stderr, flush=True)
    inputs = workload_inputs(w, seed=args.seed, device=str(dev))
    if w.varlen:
        q, k, v, beta, cu, S0, lengths = inputs
        n_tokens = int(sum(lengths))
        n_units = w.N * w.H
        order = dn.longest_first_order(cu)
        o = torch.empty_like(v)
        Sf = torch.empty((w.N, w.H, w.dv, w.dk), dtype=torch.float32, device=dev)
        g = make_gates((n_tokens, w.H), seed=args.seed, device=str(dev))

        def step(gated=args.gated):
            if gated:
                dn.deltanet_gated_fwd_varlen(q, k, v, beta, g, cu, S0, seq_order=order, o=o,
                                             S_final=Sf)
            else:
                dn.deltanet_fwd_varlen(q, k, v, beta, cu, S0, seq_order=order, o=o, S_final=Sf)
        config = {"workload": w.name, "N": w.N, "H": w.H, "total_T": n_tokens, "dk": w.dk,
                  "dv": w.dv, "chunk": w.chunk, "len_range": [w.len_lo, w.len_hi]}
        groups = 1
    else:
        q, k, v, beta, S0 = inputs
        n_tokens = w.B * w.T
        n_units = w.B * w.H
        o = torch.empty_like(v)
        Sf = torch.empty((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device=dev)
        need = dn.deltanet_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, w.chunk, args.cp_groups)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        groups = (args.cp_groups if args.cp_groups > 0 else
                  dn.deltanet_pick_cp_groups(w.B, w.H, w.T, w.dk, w.dv, w.chunk))

        g = make_gates((w.B, w.T, w.H), seed=args.seed, device=str(dev))

        def step(gated=args.gated):
            if gated:
                dn.deltanet_gated_fwd(q, k, v, beta, g, S0, o=o, S_final=Sf,
                                      cp_groups=args.cp_groups, workspace=ws)
            else:
                dn.deltanet_fwd(q, k, v, beta, S0, o=o, S_final=Sf, cp_groups=args.cp_groups,
                                workspace=ws)
        config = {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv,
                  "chunk": w.chunk, "cp_groups": groups}
    torch.cuda.synchronize()

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    print(f"[bench] warmup {args.warmup}, timing {args.steps} steps"
          f"{' (gated)' if args.gated else ''}", file=sys.stderr, flush=True)
    ms_per_step, avg_launch_ms, wall = time_steps(step, args.warmup, args.steps)
    if not bool(torch.isfinite(o).all()) or not bool(torch.isfinite(Sf).all()):
        print("bench.py: non-finite output", file=sys.stderr)
        sys.exit(3)

    tokens_per_s = n_tokens / (ms_per_step / 1e3)
    head_tokens = n_tokens * w.H
    flops = head_tokens * flops_per_head_token(w.chunk, w.dk, w.dv)
    peak_flops = PEAK_BF16_FLOPS if w.dtype == "bf16" else PEAK_FP32_FLOPS
    nbytes = algorithmic_bytes(w, esz, n_tokens, n_units, S0 is not None, True, args.gated)
    mfma_frac = flops / (ms_per_step / 1e3) / peak_flops

    # Dominant kernel: the serial path is one launch per step; with context
    # parallelism the step holds three launches and the events cover all of
    # them, so the figure is then a whole-step rate.
    achieved_gbps = nbytes / (avg_launch_ms / 1e3) / 1e9
    traffic = load_traffic(w.name, args.gated) if groups == 1 else None
    kname = ("chain_kernel_ws<128,128,out,gated>" if args.gated else "chain_kernel_ws<128,128,out>") \
        if w.dtype == "bf16" and w.dk == 128 and w.dv == 128 else "chain_kernel"
    roofline = {"bound": "hbm", "achieved": round(achieved_gbps, 1), "peak": PEAK_HBM_BPS / 1e9,
                "unit": "GB/s", "frac": round(achieved_gbps * 1e9 / PEAK_HBM_BPS, 4),
                "traffic": traffic, "kernel": kname,
                "algorithmic_bytes": nbytes, "avg_launch_us": round(avg_launch_ms * 1e3, 2),
                "mfma_tflops": round(flops / (avg_launch_ms / 1e3) / 1e12, 1),
                "mfma_frac": round(flops / (avg_launch_ms / 1e3) / peak_flops, 4)}

    metric = metric_for(w)
    result = {
        "metric": ("Gated DeltaNet " + metric) if args.gated else metric,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": config,
        "mfma_frac_of_bf16_peak": round(mfma_frac, 4),
        "mfma_frac_triangle_aware": round(head_tokens * flops_per_head_token_triangular(w.chunk, w.dk, w.dv)
                                          / (ms_per_step / 1e3) / peak_flops, 4),
        "head_tokens_per_s": round(head_tokens / (ms_per_step / 1e3), 1),
        "flops_per_step": flops,
        "wall_s_timed": round(wall, 4),
        "settle_s_untimed": SETTLE_S,
        "roofline": roofline,
    }
    def want(name):
        return not args.gated and not args.no_variants and (args.variants == "all" or name in args.variants.split(","))

    if want("gated"):
        # the same workload through deltanet_gated_fwd (log decays drawn as in synth.make_gates)
        print("[bench] gated variant: warmup 5, timing 20 steps", file=sys.stderr, flush=True)
        g_ms, g_launch_ms, _ = time_steps(lambda: step(gated=True), 5, 20)
        g_bytes = algorithmic_bytes(w, esz, n_tokens, n_units, S0 is not None, True, True)
        result.setdefault("variants", {})["gated"] = {
            "call": "deltanet_gated_fwd", "steps": 20, "warmup": 5,
            "ms_per_step": round(g_ms, 5), "tokens_per_s": round(n_tokens / (g_ms / 1e3), 1),
            "avg_launch_us": round(g_launch_ms * 1e3, 2), "algorithmic_bytes": g_bytes,
            "hbm_frac": round(g_bytes / (g_launch_ms / 1e3) / PEAK_HBM_BPS, 4),
            "mfma_frac": round(flops / (g_launch_ms / 1e3) / peak_flops, 4),
            "vs_ungated_time": round(g_launch_ms / avg_launch_ms, 4)}
    if not w.varlen and w.dtype == "bf16" and any(map(want, ("bwd", "gated_bwd", "gdp", "gdp_bwd", "kda", "kda_long",
                                                               "gated_long", "bwd_long"))):
        var = result.setdefault("variants", {})
        if want("bwd"):
            var["bwd"] = bwd_variant(dev, w, inputs, avg_launch_ms)
        if want("gated_bwd"):
            var["gated_bwd"] = gated_bwd_variant(dev, w, inputs, avg_launch_ms)
        if want("gdp") or want("gdp_bwd"):
            var["gdp"] = gdp_variant(dev, w, flops / n_tokens / w.H, peak_flops)
        if want("gdp_bwd"):
            var["gdp_bwd"] = gdp_bwd_variant(dev, w, var["gdp"]["avg_launch_us"] / 1e3)
        if want("kda"):
            var["kda"] = kda_variant(dev, w, inputs, avg_launch_ms)
        if want("kda_long"):
            var["kda_long"] = kda_long_variant(dev)
        if want("gated_long"):
            var["gated_long"] = gated_long_variant(dev)
        if want("bwd_long"):
            var["bwd_long"] = bwd_long_variant(dev)
    if want("workloads") and w.name == "layer_b8_h16_t4096":
        # the other workloads of the forward pass, each timed by the same clock
        result.setdefault("variants", {})
        result["variants"]["chunks128_b4_h16_t8192"] = workload_variant(dev, "chunks128_b4_h16_t8192", (1, 0))
        result["variants"]["long_b1_h16_t131072"] = workload_variant(dev, "long_b1_h16_t131072", (1, 0),
                                                                     steps=5, warmup=2)
        result["variants"]["varlen_n64_h32"] = workload_variant(dev, "varlen_n64_h32", steps=5, warmup=2)
        result["variants"]["tiny_f32"] = workload_variant(dev, "tiny_f32", steps=20, warmup=5)
    if want("decode"):
        result.setdefault("variants", {})["decode"] = decode_variant(dev)
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on the host", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(inputs, w, w.varlen, args.cpu_budget,
                                              g if args.gated else None)
        if result["cpu_baseline"].get("value"):
            result["cpu_baseline"]["gpu_speedup"] = round(tokens_per_s / result["cpu_baseline"]["value"], 1)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
