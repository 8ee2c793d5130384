"""Decode step (one token per (sequence, head), state updated in place) vs the
fp64 oracle, through the C-ABI.

One step of the recurrence is the oracle's token-serial forward over a
single token from the given state ("Linear Attention, Visualized",
DeltaNet > "Recurrent form"; with g, "Gated DeltaNet (GDN)"; with
per-channel g, "Kimi Delta Attention (KDA)"). Cases: every (dk, dv) and
dtype, with and without decay, one step, a loop of steps against the oracle
over the same tokens, and decoding that continues from a chunkwise forward
pass. Bar: max|gpu - oracle| / max|oracle| within 2e-2
(bf16) or 1e-4 (fp32), for o and for the state.
"""

import numpy as np
import pytest
import torch

import oracle
from chunkwise_delta_rule_amd import (deltanet_decode_step, deltanet_fwd, deltanet_gated_fwd,
                                      deltanet_kda_decode_step, deltanet_kda_fwd)
from chunkwise_delta_rule_amd.synth import make_channel_gates, make_gates, make_inputs
from helpers import TOL, f64, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _ref(q, k, v, beta, g, S0):
    if g is None:
        return oracle.deltanet_fwd(q, k, v, beta, S0)
    return oracle.gated_deltanet_fwd(q, k, v, beta, g, S0)


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("bf16", 64, 128), ("bf16", 128, 64),
                                         ("bf16", 64, 64), ("f32", 128, 128), ("f32", 64, 64)])
@pytest.mark.parametrize("gated", [False, True])
def test_decode_one_step(dtype, dk, dv, gated):
    print(f"[case] decode one step {dtype} dk={dk} dv={dv} gated={gated}", flush=True)
    B, H = 3, 5
    q, k, v, beta, S0 = make_inputs(B, H, 1, dk, dv, dtype=dtype, seed=200, s0_std=0.5)
    g = make_gates((B, 1, H), seed=200) if gated else None
    S = S0.to(DEV).clone()
    o = deltanet_decode_step(*(x[:, 0].to(DEV) for x in (q, k, v, beta)), S,
                             None if g is None else g[:, 0].to(DEV))
    torch.cuda.synchronize()
    ro, rs = _ref(f64(q), f64(k), f64(v), f64(beta), f64(g), f64(S0))
    eo, es = rel_err(f64(o), ro[:, 0]), rel_err(f64(S), rs)
    tol = TOL[q.dtype]
    print(f"  err o={eo:.3e} S={es:.3e} (tol {tol})", flush=True)
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("gated", [False, True])
def test_decode_loop_matches_recurrence(gated):
    # 100 steps from a random state, one token at a time, against the oracle over the 100 tokens
    B, H, T = 2, 4, 100
    print(f"[case] decode loop T={T} gated={gated}", flush=True)
    q, k, v, beta, S0 = make_inputs(B, H, T, 128, 128, seed=201, s0_std=0.3)
    g = make_gates((B, T, H), seed=201) if gated else None
    d = [x.to(DEV) for x in (q, k, v, beta)]
    dg = None if g is None else g.to(DEV)
    S = S0.to(DEV).clone()
    outs = []
    for t in range(T):
        outs.append(deltanet_decode_step(*(x[:, t].contiguous() for x in d), S,
                                         None if dg is None else dg[:, t].contiguous()))
    torch.cuda.synchronize()
    o = torch.stack(outs, dim=1)
    ro, rs = _ref(f64(q), f64(k), f64(v), f64(beta), f64(g), f64(S0))
    eo, es = rel_err(f64(o), ro), rel_err(f64(S), rs)
    print(f"  err o={eo:.3e} S={es:.3e}", flush=True)
    assert eo <= 2e-2 and es <= 2e-2


@pytest.mark.parametrize("gated", [False, True])
def test_decode_continues_a_forward_pass(gated):
    # prefill 300 tokens chunkwise, then decode 20 more from the returned state
    B, H, T0, T1 = 2, 3, 300, 20
    print(f"[case] prefill {T0} + decode {T1} gated={gated}", flush=True)
    q, k, v, beta, S0 = make_inputs(B, H, T0 + T1, 128, 128, seed=202, s0_std=0.2)
    g = make_gates((B, T0 + T1, H), seed=202) if gated else None
    d = [x.to(DEV) for x in (q, k, v, beta)]
    dg = None if g is None else g.to(DEV)
    pre = [x[:, :T0].contiguous() for x in d]
    if gated:
        o_pre, S = deltanet_gated_fwd(*pre, dg[:, :T0].contiguous(), S0.to(DEV))
    else:
        o_pre, S = deltanet_fwd(*pre, S0.to(DEV))
    outs = []
    for t in range(T0, T0 + T1):
        outs.append(deltanet_decode_step(*(x[:, t].contiguous() for x in d), S,
                                         None if dg is None else dg[:, t].contiguous()))
    torch.cuda.synchronize()
    o = np.concatenate([f64(o_pre), f64(torch.stack(outs, dim=1))], axis=1)
    ro, rs = _ref(f64(q), f64(k), f64(v), f64(beta), f64(g), f64(S0))
    eo, es = rel_err(o, ro), rel_err(f64(S), rs)
    print(f"  err o={eo:.3e} S={es:.3e}", flush=True)
    assert eo <= 2e-2 and es <= 2e-2


# ---- Kimi Delta Attention decode: per-channel decay ("Linear Attention,
# Visualized", "Kimi Delta Attention (KDA)"), against the oracle's token-serial
# KDA forward over the same tokens.

@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("bf16", 64, 128), ("bf16", 128, 64),
                                         ("bf16", 64, 64), ("f32", 128, 128), ("f32", 64, 64)])
def test_kda_decode_one_step(dtype, dk, dv):
    print(f"[case] kda decode one step {dtype} dk={dk} dv={dv}", flush=True)
    B, H = 3, 5
    q, k, v, beta, S0 = make_inputs(B, H, 1, dk, dv, dtype=dtype, seed=210, s0_std=0.5)
    g = make_channel_gates((B, 1, H, dk), seed=210)
    S = S0.to(DEV).clone()
    o = deltanet_kda_decode_step(*(x[:, 0].to(DEV) for x in (q, k, v, beta)), S, g[:, 0].to(DEV))
    torch.cuda.synchronize()
    ro, rs = oracle.kda_fwd(f64(q), f64(k), f64(v), f64(beta), f64(g), f64(S0))
    eo, es = rel_err(f64(o), ro[:, 0]), rel_err(f64(S), rs)
    tol = TOL[q.dtype]
    print(f"  err o={eo:.3e} S={es:.3e} (tol {tol})", flush=True)
    assert eo <= tol and es <= tol


def test_kda_decode_continues_a_forward_pass():
    # prefill 200 tokens with the chunkwise KDA kernel, then decode 20 more
    B, H, T0, T1 = 2, 3, 200, 20
    print(f"[case] kda prefill {T0} + decode {T1}", flush=True)
    q, k, v, beta, S0 = make_inputs(B, H, T0 + T1, 128, 128, seed=211, s0_std=0.2)
    g = make_channel_gates((B, T0 + T1, H, 128), seed=211)
    d = [x.to(DEV) for x in (q, k, v, beta)]
    dg = g.to(DEV)
    o_pre, S = deltanet_kda_fwd(*(x[:, :T0].contiguous() for x in d), dg[:, :T0].contiguous(), S0.to(DEV))
    outs = []
    for t in range(T0, T0 + T1):
        outs.append(deltanet_kda_decode_step(*(x[:, t].contiguous() for x in d), S, dg[:, t].contiguous()))
    torch.cuda.synchronize()
    o = np.concatenate([f64(o_pre), f64(torch.stack(outs, dim=1))], axis=1)
    ro, rs = oracle.kda_fwd(f64(q), f64(k), f64(v), f64(beta), f64(g), f64(S0))
    eo, es = rel_err(o, ro), rel_err(f64(S), rs)
    print(f"  err o={eo:.3e} S={es:.3e}", flush=True)
    assert eo <= 2e-2 and es <= 2e-2
