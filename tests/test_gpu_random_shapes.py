"""Seeded random configurations of the forward entry points against the oracle.

Each case draws its shape, widths, dtype, context-parallel group count,
initial state and decay strength from a fixed-seed generator, so the set is
the same on every run; the case line is printed before the GPU call. The
draws cover what the fixed cases cover one axis at a time, in combination:
ragged lengths from 1 to 1200 tokens, unit counts off the block map's groups
of 8, forced and automatic group counts (including one chunk per group), the
32-, 64- and 128-row tile layouts, and packed batches with empty sequences.
Bar as in the other parity tests: max|gpu - oracle| / max|oracle| <= 2e-2
(bf16 inputs) or 1e-4 (fp32), for o and for the final state separately.
"""

import numpy as np
import pytest
import torch

import oracle
import chunkwise_delta_rule_amd as dn
from chunkwise_delta_rule_amd.synth import make_channel_gates, make_gates, make_inputs, make_varlen_inputs
from helpers import TOL, f64, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def draw_dense(i):
    r = np.random.default_rng(1000 + i)
    fp32 = r.random() < 0.15
    dk = 64 if fp32 else int(r.choice([64, 128], p=[0.35, 0.65]))
    dv = int(r.choice([64, 128], p=[0.35, 0.65]))
    B, H = int(r.integers(1, 4)), int(r.integers(1, 6))
    T = int(r.integers(1, 1200))
    nc = (T + 63) // 64
    cp = int(r.choice([1, 0, int(r.integers(2, max(3, nc + 1)))]))
    s0 = float(r.choice([0.0, 0.3]))
    mu = float(r.choice([-1.0, 2.0, 5.0]))
    return dict(B=B, H=H, T=T, dk=dk, dv=dv, dtype="f32" if fp32 else "bf16", cp=cp, s0=s0, mu=mu)


def check(o, Sf, ro, rs, dt):
    tol = TOL[dt]
    eo, es = rel_err(f64(o), ro), rel_err(f64(Sf), rs)
    print(f"  err o={eo:.3e} S={es:.3e} (tol {tol})", flush=True)
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("i", range(12))
def test_random_deltanet_fwd(i):
    c = draw_dense(i)
    print(f"[case] deltanet_fwd {c}", flush=True)
    q, k, v, beta, S0 = make_inputs(c["B"], c["H"], c["T"], c["dk"], c["dv"], dtype=c["dtype"], seed=2000 + i,
                                    s0_std=c["s0"])
    o, Sf = dn.deltanet_fwd(*(x.to(DEV) for x in (q, k, v, beta)), None if S0 is None else S0.to(DEV),
                            cp_groups=c["cp"])
    torch.cuda.synchronize()
    ro, rs = oracle.deltanet_fwd(f64(q), f64(k), f64(v), f64(beta), f64(S0))
    check(o, Sf, ro, rs, q.dtype)


@pytest.mark.parametrize("i", range(12, 22))
def test_random_gated_fwd(i):
    c = draw_dense(i)
    print(f"[case] deltanet_gated_fwd {c}", flush=True)
    q, k, v, beta, S0 = make_inputs(c["B"], c["H"], c["T"], c["dk"], c["dv"], dtype=c["dtype"], seed=2000 + i,
                                    s0_std=c["s0"])
    g = make_gates((c["B"], c["T"], c["H"]), seed=2000 + i, mu=c["mu"])
    o, Sf = dn.deltanet_gated_fwd(*(x.to(DEV) for x in (q, k, v, beta, g)), None if S0 is None else S0.to(DEV),
                                  cp_groups=c["cp"])
    torch.cuda.synchronize()
    ro, rs = oracle.gated_deltanet_fwd(f64(q), f64(k), f64(v), f64(beta), f64(g), f64(S0))
    check(o, Sf, ro, rs, q.dtype)


@pytest.mark.parametrize("i", range(22, 30))
def test_random_kda_fwd(i):
    c = draw_dense(i)
    c["dtype"] = "bf16"  # the KDA kernel takes bf16 only
    print(f"[case] deltanet_kda_fwd {c}", flush=True)
    q, k, v, beta, S0 = make_inputs(c["B"], c["H"], c["T"], c["dk"], c["dv"], dtype="bf16", seed=2000 + i,
                                    s0_std=c["s0"])
    g = make_channel_gates((c["B"], c["T"], c["H"], c["dk"]), seed=2000 + i, mu=c["mu"])
    o, Sf = dn.deltanet_kda_fwd(*(x.to(DEV) for x in (q, k, v, beta, g)), None if S0 is None else S0.to(DEV),
                                cp_groups=c["cp"])
    torch.cuda.synchronize()
    ro, rs = oracle.kda_fwd(f64(q), f64(k), f64(v), f64(beta), f64(g), f64(S0))
    check(o, Sf, ro, rs, q.dtype)


@pytest.mark.parametrize("i", range(30, 36))
def test_random_varlen_fwd(i):
    r = np.random.default_rng(1000 + i)
    N = int(r.integers(1, 9))
    lengths = [int(x) for x in r.integers(0, 400, size=N)]
    if N > 2:
        lengths[int(r.integers(0, N))] = 0  # an empty sequence
    H = int(r.integers(1, 5))
    dk, dv = int(r.choice([64, 128])), int(r.choice([64, 128]))
    s0 = float(r.choice([0.0, 0.3]))
    gated = bool(r.random() < 0.5)
    print(f"[case] varlen lengths={lengths} H={H} dk={dk} dv={dv} s0={s0} gated={gated}", flush=True)
    q, k, v, beta, cu, S0 = make_varlen_inputs(lengths, H, dk, dv, seed=3000 + i, s0_std=s0)
    d = [x.to(DEV) for x in (q, k, v, beta)]
    dS0 = None if S0 is None else S0.to(DEV)
    order = dn.longest_first_order(cu.to(DEV))
    if gated:
        g = make_gates((q.shape[0], H), seed=3000 + i, mu=float(r.choice([-1.0, 2.0])))
        o, Sf = dn.deltanet_gated_fwd_varlen(*d, g.to(DEV), cu.to(DEV), dS0, seq_order=order)
        torch.cuda.synchronize()
        ro, rs = oracle.gated_deltanet_fwd_varlen(f64(q), f64(k), f64(v), f64(beta), f64(g), cu.numpy(), f64(S0))
    else:
        o, Sf = dn.deltanet_fwd_varlen(*d, cu.to(DEV), dS0, seq_order=order)
        torch.cuda.synchronize()
        ro, rs = oracle.deltanet_fwd_varlen(f64(q), f64(k), f64(v), f64(beta), cu.numpy(), f64(S0))
    check(o, Sf, ro, rs, q.dtype)
